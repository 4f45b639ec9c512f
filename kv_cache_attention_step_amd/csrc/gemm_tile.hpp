// bf16 "TN" GEMM main loop for gfx950: C[M, N] = A[M, K] . B[N, K]^T with both
// operands K-contiguous, fp32 accumulation in MFMA registers.
//
// Block tile BM x BN x 64, 256 threads = 4 waves arranged 2 x 2, each wave owning
// a (BM/2) x (BN/2) tile held as (BM/64) x (BN/64) accumulators of
// v_mfma_f32_32x32x16_bf16. Tiles are staged through LDS, double buffered: while
// the MFMAs consume stage s, the next K-slice is already in flight from global
// memory into registers and is written to stage s^1 afterwards (one barrier per
// K-slice). Within a stage a row of 64 bf16 is eight 16-byte chunks; chunk c of
// row r sits at chunk position c ^ (r & 7), so the 32 rows a fragment read
// touches spread over all LDS banks.
#pragma once
#include "fc_common.hpp"

template <int BM, int BN>
struct GemmCfg {
  static constexpr int BK = 64;
  static constexpr int WM = BM / 2, WN = BN / 2;
  static constexpr int MB = WM / 32, NB = WN / 32;
  static constexpr int A_BYTES = BM * BK * 2;
  static constexpr int B_BYTES = BN * BK * 2;
  static constexpr int STAGE = A_BYTES + B_BYTES;
  static constexpr int LDS_BYTES = 2 * STAGE;
  static constexpr int A_LD = BM * 8 / 256;  // 16-byte chunks per thread per stage
  static constexpr int B_LD = BN * 8 / 256;
  static_assert(BM % 64 == 0 && BN % 64 == 0, "tile");
};

FC_DEVICE int swz_off(int row, int chunk) { return (row * 8 + (chunk ^ (row & 7))) * 16; }

template <int BM, int BN>
struct GemmMainloop {
  using C = GemmCfg<BM, BN>;

  // Loads one K-slice of A (rows m0..) and B (rows n0..) through buffer
  // descriptors whose range ends at row M (resp. N): rows past the end read 0.
  static FC_DEVICE void load(__amdgpu_buffer_rsrc_t ra_desc, int lda, __amdgpu_buffer_rsrc_t rb_desc,
                             int ldb, int m0, int n0, int k0, u32x4_t (&ra)[C::A_LD],
                             u32x4_t (&rb)[C::B_LD]) {
    const int t = threadIdx.x;
    const int c = t & 7;
#pragma unroll
    for (int i = 0; i < C::A_LD; ++i) {
      const int r = (t >> 3) + 32 * i;
      ra[i] = __builtin_amdgcn_raw_buffer_load_b128(ra_desc, ((m0 + r) * lda + k0 + c * 8) * 2, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < C::B_LD; ++i) {
      const int r = (t >> 3) + 32 * i;
      rb[i] = __builtin_amdgcn_raw_buffer_load_b128(rb_desc, ((n0 + r) * ldb + k0 + c * 8) * 2, 0, 0);
    }
  }

  static FC_DEVICE void store(char* stage, const u32x4_t (&ra)[C::A_LD],
                              const u32x4_t (&rb)[C::B_LD]) {
    const int t = threadIdx.x;
    const int c = t & 7;
#pragma unroll
    for (int i = 0; i < C::A_LD; ++i) {
      const int r = (t >> 3) + 32 * i;
      *(u32x4_t*)(stage + swz_off(r, c)) = ra[i];
    }
    char* sb = stage + C::A_BYTES;
#pragma unroll
    for (int i = 0; i < C::B_LD; ++i) {
      const int r = (t >> 3) + 32 * i;
      *(u32x4_t*)(sb + swz_off(r, c)) = rb[i];
    }
  }

  static FC_DEVICE void compute(const char* stage, int wm, int wn,
                                f32x16_t (&acc)[C::MB][C::NB]) {
    const int lane = threadIdx.x & 63;
    const int lr = lane & 31, hb = lane >> 5;
    const char* sa = stage;
    const char* sb = stage + C::A_BYTES;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const int chunk = kk * 2 + hb;
      bf16x8_t af[C::MB], bfr[C::NB];
#pragma unroll
      for (int mb = 0; mb < C::MB; ++mb) {
        const int r = wm * C::WM + mb * 32 + lr;
        af[mb] = as_bf16x8(*(const u32x4_t*)(sa + swz_off(r, chunk)));
      }
#pragma unroll
      for (int nb = 0; nb < C::NB; ++nb) {
        const int r = wn * C::WN + nb * 32 + lr;
        bfr[nb] = as_bf16x8(*(const u32x4_t*)(sb + swz_off(r, chunk)));
      }
#pragma unroll
      for (int mb = 0; mb < C::MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < C::NB; ++nb) acc[mb][nb] = mfma32x32x16(af[mb], bfr[nb], acc[mb][nb]);
    }
  }

  // Full K loop. K must be a multiple of 64 and M*lda*2, N*ldb*2 < 2^31.
  // Leaves LDS free (ends on a barrier).
  static FC_DEVICE void run(const uint16_t* __restrict__ A, int lda, int M,
                            const uint16_t* __restrict__ Bm, int ldb, int N, int K, int m0, int n0,
                            char* lds, f32x16_t (&acc)[C::MB][C::NB]) {
    const int wave = threadIdx.x >> 6;
    const int wm = wave >> 1, wn = wave & 1;
#pragma unroll
    for (int mb = 0; mb < C::MB; ++mb)
#pragma unroll
      for (int nb = 0; nb < C::NB; ++nb)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[mb][nb][i] = 0.f;

    u32x4_t ra[C::A_LD], rb[C::B_LD];
    const int KT = K / C::BK;
    const __amdgpu_buffer_rsrc_t da = make_rsrc(A, (uint32_t)M * lda * 2);
    const __amdgpu_buffer_rsrc_t db = make_rsrc(Bm, (uint32_t)N * ldb * 2);
    load(da, lda, db, ldb, m0, n0, 0, ra, rb);
    store(lds, ra, rb);
    __syncthreads();
    for (int kt = 0; kt < KT; ++kt) {
      const bool more = kt + 1 < KT;
      if (more) load(da, lda, db, ldb, m0, n0, (kt + 1) * C::BK, ra, rb);
      compute(lds + (kt & 1) * C::STAGE, wm, wn, acc);
      if (more) store(lds + ((kt + 1) & 1) * C::STAGE, ra, rb);
      __syncthreads();
    }
  }
};

// Output coordinates of accumulator register i of block (mb, nb) for this lane,
// relative to the wave tile.
FC_DEVICE int acc_row(int mb, int i, int lane) { return mb * 32 + (i >> 2) * 8 + (lane >> 5) * 4 + (i & 3); }
FC_DEVICE int acc_col(int nb, int lane) { return nb * 32 + (lane & 31); }
