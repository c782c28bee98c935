// Host-only checks of the packed weight orders the kernels and the export
// paths share (csrc/frt_device.h, csrc/frt_qkv_dev.h, csrc/frt_mx.h): every order is a
// bijection onto its packed range, and keeps together what its kernel needs
// together.  Built with hipcc and run on the CPU by tests/test_layouts_cpu.py
// (no GPU call is made).  Exit status 0 when every check holds.
#include "frt_qkv_dev.h"
#include "frt_mx.h"

#include <cstdio>
#include <vector>

using namespace frt;

static int fails = 0;
#define CHECK(cond, ...)            \
  do {                              \
    if (!(cond)) {                  \
      std::printf(__VA_ARGS__);     \
      std::printf("\n");            \
      ++fails;                      \
    }                               \
  } while (0)

// packed_offset: [N][K] onto N*K bytes, 16 consecutive K values of a row
// contiguous
static void check_packed(uint32_t N, uint32_t K) {
  std::vector<int> seen((size_t)N * K, 0);
  for (uint32_t n = 0; n < N; ++n)
    for (uint32_t k = 0; k < K; ++k) {
      const size_t o = packed_offset(n, k, K);
      CHECK(o < seen.size() && seen[o]++ == 0, "packed_offset(%u, %u, %u) = %zu", n, k, K, o);
      if (k % 16) CHECK(o == packed_offset(n, k - 1, K) + 1, "packed_offset not contiguous at %u %u", n, k);
    }
}

// quad_offset: a bijection; quad q's bytes are [4qK, 4(q+1)K); in block t
// lane l holds column 4q + (l & 3), K part (l & 15) >> 2, elements
// 256t + 64p + (l >> 4)*16 .. + 15
static void check_quad(uint32_t N, uint32_t K) {
  std::vector<int> seen((size_t)N * K, 0);
  for (uint32_t n = 0; n < N; ++n)
    for (uint32_t k = 0; k < K; ++k) {
      const size_t o = quad_offset(n, k, K);
      CHECK(o < seen.size() && seen[o]++ == 0, "quad_offset(%u, %u, %u) = %zu", n, k, K, o);
      const size_t q = n / 4;
      CHECK(o >= q * 4 * K && o < (q + 1) * 4 * K, "quad_offset(%u, %u) outside its quad's range", n, k);
      const uint32_t t = k / 256, p = (k % 256) / 64, kk = k % 64;
      const size_t lane = (kk / 16) * 16 + p * 4 + (n % 4);
      CHECK(o == (((size_t)q * (K / 256) + t) * 64 + lane) * 16 + (k % 16), "quad_offset(%u, %u) lane order", n, k);
    }
}

// the gated gate/up orders: gate i and up i onto distinct rows of [0, 2I);
// 16 + 16 order: gate and up of 16 columns in consecutive 16-row groups;
// octet order: gate and up of column i in one group, 8 rows apart
static void check_gated(uint32_t I) {
  std::vector<int> a(2 * I, 0), b(2 * I, 0);
  for (uint32_t i = 0; i < I; ++i) {
    const uint32_t g = gate_row(i), u = up_row_gated(i);
    CHECK(g < 2 * I && u < 2 * I && a[g]++ == 0 && a[u]++ == 0, "gate_row / up_row_gated collide at %u", i);
    CHECK(u == g + 16 && (g / 16) % 2 == 0, "16 + 16 order at %u", i);
    const uint32_t go = gate_row_oct(i), uo = up_row_oct(i);
    CHECK(go < 2 * I && uo < 2 * I && b[go]++ == 0 && b[uo]++ == 0, "octet rows collide at %u", i);
    CHECK(uo == go + 8 && go / 16 == uo / 16 && go % 16 < 8, "octet order at %u", i);
  }
}

// the fused QKV orders: [q; k; v] rows onto [0, N); pairs and octets keep
// every rotation pair (d, d + hd/2) of a q or k head in one lane row of
// two groups (pairs: 16 rows apart) or of one group (octets: 8 rows apart)
static void check_qkv(uint32_t nq, uint32_t nkv, uint32_t hd) {
  const uint32_t N = (nq + 2 * nkv) * hd, n_rope = (nq + nkv) * hd, half = hd / 2;
  std::vector<int> a(N, 0), b(N, 0);
  for (uint32_t n = 0; n < N; ++n) {
    const uint32_t p = qkv_packed_row(n, hd, n_rope), o = qkv_packed_row_oct(n, hd, n_rope);
    CHECK(p < N && a[p]++ == 0, "qkv_packed_row collides at %u (nq %u nkv %u hd %u)", n, nq, nkv, hd);
    CHECK(o < N && b[o]++ == 0, "qkv_packed_row_oct collides at %u (nq %u nkv %u hd %u)", n, nq, nkv, hd);
    if (n < n_rope && (n % hd) < half) {
      const uint32_t m = n + half;  // the rotation partner
      CHECK(qkv_packed_row(m, hd, n_rope) == p + 16, "pair order splits the rotation pair at %u", n);
      CHECK(qkv_packed_row_oct(m, hd, n_rope) == o + 8 && o % 16 < 8, "octet order splits the pair at %u", n);
    }
    if (n >= n_rope) CHECK(o == n, "v row %u moved in the octet order", n);
  }
}

// MXFP4 orders, per 32-value block b of row n.  GEMV order: 16-row groups,
// 1 KiB per (group, 128-K block), exponents per (group, four K blocks).
// Column-quad order (the whole-column down GEMV): quad q's codes in
// [q K/2 * 4, (q + 1) K/2 * 4) and exponents in [q K/8, (q + 1) K/8); in step
// t lane l holds column 4q + l % 4, part p = (l % 16) / 4, sub-block l / 16,
// the block 16t + 4p + l / 16; the activation exponent the kernel reads for
// row m < 4 and that block is byte p of dword 64t + 16 (l / 16) + m of the
// HQ slot's GEMV layout.
static void check_mx(uint32_t N, uint32_t K) {
  const uint32_t nb = K / 32, KB = K / 128;
  std::vector<int> c1(N * nb, 0), s1(N * nb, 0), c2(N * nb, 0), s2(N * nb, 0);
  for (uint32_t n = 0; n < N; ++n)
    for (uint32_t b = 0; b < nb; ++b) {
      const uint32_t kb = b / 4, lane = (n % 16) + 16 * (b % 4);
      const size_t co = mx_code_off(n, kb, lane, KB), so = mx_scale_off(n, kb, lane, KB);
      CHECK(co % 16 == 0 && co / 16 < c1.size() && c1[co / 16]++ == 0, "mx_code_off(%u, %u, K %u) = %zu", n, b, K, co);
      CHECK(so < s1.size() && s1[so]++ == 0, "mx_scale_off(%u, %u, K %u) = %zu", n, b, K, so);
      const size_t qc = mx_quad_code_off(n, b, K), qs = mx_quad_scale_off(n, b, K);
      CHECK(qc % 16 == 0 && qc / 16 < c2.size() && c2[qc / 16]++ == 0, "mx_quad_code_off(%u, %u, K %u) = %zu", n, b,
            K, qc);
      CHECK(qs < s2.size() && s2[qs]++ == 0, "mx_quad_scale_off(%u, %u, K %u) = %zu", n, b, K, qs);
      const size_t q = n / 4;
      CHECK(qc >= q * 2 * K && qc < (q + 1) * 2 * K, "mx_quad_code_off(%u, %u) outside its quad", n, b);
      const uint32_t t = b / 16, p = (b % 16) / 4, sb = b % 4, l = sb * 16 + p * 4 + n % 4;
      CHECK(qc == (((size_t)q * (K / 512) + t) * 64 + l) * 16 && qs == ((size_t)q * (K / 512) + t) * 64 + l,
            "column-quad lane order at %u %u", n, b);
      if (n < 4)
        CHECK(mx_act_scale_off_gemv(n, b, KB) == ((size_t)t * 64 + sb * 16 + n) * 4 + p,
              "activation exponent of row %u block %u", n, b);
    }
}

int main() {
  for (uint32_t N : {16u, 48u}) for (uint32_t K : {128u, 384u}) check_packed(N, K);
  for (uint32_t N : {4u, 12u, 40u}) for (uint32_t K : {256u, 768u, 1280u}) check_quad(N, K);
  for (uint32_t I : {16u, 48u, 128u, 640u}) check_gated(I);
  for (uint32_t N : {16u, 48u}) for (uint32_t K : {512u, 1536u, 2560u}) check_mx(N, K);
  check_qkv(2, 1, 64);
  check_qkv(4, 2, 32);
  check_qkv(8, 1, 256);
  check_qkv(32, 8, 128);
  if (fails) {
    std::printf("%d layout checks failed\n", fails);
    return 1;
  }
  std::printf("layout checks ok\n");
  return 0;
}
