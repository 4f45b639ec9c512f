// bf16 "TN" GEMM main loop for gfx950: C[M, N] = A[M, K] . B[N, K]^T with both
// operands K-contiguous, fp32 accumulation in MFMA registers.
//
// Block tile BM x BN x 64, 256 threads = 4 waves arranged 2 x 2, each wave owning
// a (BM/2) x (BN/2) tile held as (BM/64) x (BN/64) accumulators of
// v_mfma_f32_32x32x16_bf16. Tiles are staged through LDS, double buffered: while
// the MFMAs consume stage s, the next K-slice is already in flight from global
// memory into registers and is written to stage s^1 afterwards (one barrier per
// K-slice). Within a stage a row of 64 bf16 is eight 16-byte chunks; chunk c of
// row r sits at chunk position c ^ ((r >> 1) & 7). A 128-byte row covers half
// of the 64 LDS banks, so a 16-lane phase of a fragment read (16 consecutive
// rows, one logical chunk) lands on 16 distinct (row parity, chunk) bank groups.
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

FC_DEVICE int swz_off(int row, int chunk) { return (row * 8 + (chunk ^ ((row >> 1) & 7))) * 16; }

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
    // the prefetch of slice kt+1 is unconditional (past K it reads in-range rows
    // or zeros and is never consumed) so the compiler's wait counts stay exact
    for (int kt = 0; kt < KT; ++kt) {
      load(da, lda, db, ldb, m0, n0, (kt + 1) * C::BK, ra, rb);
      compute(lds + (kt & 1) * C::STAGE, wm, wn, acc);
      store(lds + ((kt + 1) & 1) * C::STAGE, ra, rb);
      __syncthreads();
    }
  }
};

// Output coordinates of accumulator register i of block (mb, nb) for this lane,
// relative to the wave tile.
FC_DEVICE int acc_row(int mb, int i, int lane) { return mb * 32 + (i >> 2) * 8 + (lane >> 5) * 4 + (i & 3); }
FC_DEVICE int acc_col(int nb, int lane) { return nb * 32 + (lane & 31); }

// ---------------------------------------------------------------------------
// 8-wave variant for large projections: 256 x 256 x 64 tile, 512 threads, two
// waves per SIMD. Waves form a 2 (rows) x 4 (column groups) grid; each owns 128
// rows x 64 columns = 4 x 2 accumulator blocks. Global loads run two K-slices
// ahead of the MFMAs (two register sets, alternated by unrolling the K loop by
// two), so a slice's load latency is hidden behind two slices of MFMA work.
// The column group -> B row map is a template functor so an epilogue can ask
// for the columns it needs in one lane (e.g. RoPE partners e and e + 64).
// ---------------------------------------------------------------------------
struct ColsLinear {  // wave column group wn, block nb -> tile column
  static FC_DEVICE int col(int wn, int nb, int lr) { return wn * 64 + nb * 32 + lr; }
};
// Column group wn covers half (wn & 1) of head (wn >> 1) of a 128-wide head:
// block 0 = head columns 32*half + [0, 32), block 1 = 64 + 32*half + [0, 32),
// so rotate-half partners (e, e + 64) share a lane and a register index.
struct ColsRopePairs {
  static FC_DEVICE int col(int wn, int nb, int lr) {
    return (wn >> 1) * 128 + nb * 64 + (wn & 1) * 32 + lr;
  }
};

template <class COLS>
struct Gemm8 {
  static constexpr int BM = 256, BN = 256, BK = 64, THREADS = 512;
  static constexpr int MB = 4, NB = 2;
  static constexpr int A_BYTES = BM * BK * 2, B_BYTES = BN * BK * 2;
  static constexpr int STAGE = A_BYTES + B_BYTES;
  static constexpr int LDS_BYTES = 2 * STAGE;
  static constexpr int LD = BM * 8 / THREADS;  // 16-byte chunks per thread per operand

  struct Regs {
    u32x4_t a[LD], b[LD];
  };

  static FC_DEVICE void load(__amdgpu_buffer_rsrc_t da, int lda, __amdgpu_buffer_rsrc_t db, int ldb,
                             int m0, int n0, int k0, Regs& r) {
    const int t = threadIdx.x;
    const int c = t & 7;
#pragma unroll
    for (int i = 0; i < LD; ++i) {
      const int row = (t >> 3) + 64 * i;
      r.a[i] = __builtin_amdgcn_raw_buffer_load_b128(da, ((m0 + row) * lda + k0 + c * 8) * 2, 0, 0);
      r.b[i] = __builtin_amdgcn_raw_buffer_load_b128(db, ((n0 + row) * ldb + k0 + c * 8) * 2, 0, 0);
    }
  }

  static FC_DEVICE void store(char* stage, const Regs& r) {
    const int t = threadIdx.x;
    const int c = t & 7;
#pragma unroll
    for (int i = 0; i < LD; ++i) {
      const int row = (t >> 3) + 64 * i;
      *(u32x4_t*)(stage + swz_off(row, c)) = r.a[i];
      *(u32x4_t*)(stage + A_BYTES + swz_off(row, c)) = r.b[i];
    }
  }

  // The MFMA cluster runs at raised wave priority: of the two waves sharing a
  // SIMD, the one feeding the matrix unit wins issue arbitration, which
  // staggers the pair so one wave's loads and barrier wait overlap the other's
  // MFMAs.
  static FC_DEVICE void compute(const char* stage, int wm, int wn, f32x16_t (&acc)[MB][NB]) {
    const int lane = threadIdx.x & 63;
    const int lr = lane & 31, hb = lane >> 5;
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const int chunk = kk * 2 + hb;
      bf16x8_t af[MB], bfr[NB];
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
        af[mb] = as_bf16x8(*(const u32x4_t*)(stage + swz_off(wm * 128 + mb * 32 + lr, chunk)));
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
        bfr[nb] = as_bf16x8(*(const u32x4_t*)(stage + A_BYTES + swz_off(COLS::col(wn, nb, lr), chunk)));
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) acc[mb][nb] = mfma32x32x16(af[mb], bfr[nb], acc[mb][nb]);
    }
    __builtin_amdgcn_s_setprio(0);
  }

  // K must be a multiple of 64. Ends on a barrier. The prefetch loads and LDS
  // stores are unconditional (slices past K read in-range rows or zeros through
  // the buffer descriptor and are never consumed): conditional loads make the
  // compiler's wait counts pessimistic and would serialise the pipeline.
  static FC_DEVICE void run(const uint16_t* __restrict__ A, int lda, int M,
                            const uint16_t* __restrict__ Bm, int ldb, int N, int K, int m0, int n0,
                            char* lds, f32x16_t (&acc)[MB][NB]) {
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = wave >> 2, wn = wave & 3;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[mb][nb][i] = 0.f;
    const __amdgpu_buffer_rsrc_t da = make_rsrc(A, (uint32_t)M * lda * 2);
    const __amdgpu_buffer_rsrc_t db = make_rsrc(Bm, (uint32_t)N * ldb * 2);
    const int KT = K / BK;
    Regs x, y;
    load(da, lda, db, ldb, m0, n0, 0, x);
    store(lds, x);
    load(da, lda, db, ldb, m0, n0, BK, x);
    load(da, lda, db, ldb, m0, n0, 2 * BK, y);
    __syncthreads();
    // at slice t (even): stage 0 holds slice t, x holds slice t+1, y slice t+2
    for (int t = 0; t < KT; t += 2) {
      compute(lds, wm, wn, acc);
      store(lds + STAGE, x);
      __syncthreads();
      load(da, lda, db, ldb, m0, n0, (t + 3) * BK, x);
      if (t + 1 < KT) compute(lds + STAGE, wm, wn, acc);
      store(lds, y);
      __syncthreads();
      load(da, lda, db, ldb, m0, n0, (t + 4) * BK, y);
    }
  }
};
