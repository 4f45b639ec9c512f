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
// 8-wave variant for large projections: BM x 256 tile (BM = 256 or 128), 512
// threads, two waves per SIMD. Waves form a 4 (rows) x 2 (columns) grid; each
// owns BM/4 rows x 128 columns = (BM/128) x 4 accumulator blocks, so a wave holds
// whole 128-wide heads: rotate-half partners e and e + 64 sit in blocks nb and
// nb + 2 of one lane, and an epilogue can write each row's 256 bytes of a head
// from one wave. The 128-row tile doubles the tile count where 256-row tiles
// would leave most of a last round of workgroups empty (M = 2048: 768 tiles
// instead of 384 over 256 CUs).
//
// Operands travel global -> LDS by the buffer unit's direct-to-LDS loads (no
// staging registers) in K-slices of 64. 128-row tiles: a stage is A (128 rows x
// 128 bytes) then B (256 rows x 128 bytes), 48 KB; three stages rotate and a
// slice is requested two slices before it is consumed. 256-row tiles: A and B
// (32 KB each per slice) have rings of their own, three A stages and two B
// stages (160 KB, all of the LDS), and every wave requests its part of B for the
// next slice in its first memory phase of a slice and its part of A for the
// slice after that in its second: each of the four phases of a slice then
// carries the same 16 KB of loads. The load path of a CU moves about 32 bytes
// per clock, so a slice's 64 KB take as long as its MFMAs; issued all in one
// memory phase per group (one shared ring), they held up those phases and the
// loop ran at 1.5 slice-times per slice; spread this way, 8 % faster. A load instruction
// moves 8 rows x 128 bytes, so every group of 8 lanes fetches one whole
// 128-byte line: L2 serves such a stream at close to twice the rate of 64-byte
// row pieces. Within a row, 16-byte chunk c sits at position c ^ ((row >> 1) & 7)
// (chosen by which chunk each lane fetches, since the DMA writes in lane order),
// so the 16 rows of a fragment-read phase land on distinct bank groups.
//
// Schedule ("ping-pong"): waves 0-3 (the first half of the tile rows) and waves
// 4-7 (the second half) put one wave of each group on every SIMD and run half a period apart,
// separated by s_barrier. In its memory phase a wave reads the fragments of one
// 32-wide half-slice (both k16 steps) and issues its refills (above) into stages
// just freed; in its compute phase it issues the 16 MFMAs of that half-slice. So one wave of each SIMD feeds the matrix unit while
// the other one waits on LDS and memory. A stage is refilled only after both
// groups have read it (the memory phase ends with lgkmcnt(0) before its barrier)
// and read only after every wave has waited for its own loads of it.
// ---------------------------------------------------------------------------

template <int BM_>
struct Gemm8 {
  static constexpr int BM = BM_, BN = 256, BK = 64, THREADS = 512;
  static constexpr int MB = BM / 128, NB = 4;
  static constexpr int WROWS = BM / 4;              // tile rows of one wave
  static constexpr int HALF_A = BM * BK * 2;        // A part of a stage
  static constexpr int HALF = BN * BK * 2;          // B part of a stage: 32 KB
  static constexpr int STAGE = HALF_A + HALF;       // bytes of an A-then-B stage (BM 128)
  static constexpr int NST = 3;                     // A-then-B stages (BM 128)
  static constexpr int DMA_N = BM / 64 + 4;         // direct-to-LDS loads per wave per slice
  static constexpr int DMA_A = BM / 64;             // of them for A
  static_assert(BM == 128 || BM == 256, "tile height");
  // 256-row tiles: separate A and B rings (3 + 2 stages of 32 KB, 160 KB);
  // 128-row tiles: three A-then-B stages of 48 KB (144 KB). LDS objects, each a
  // __shared__ array of its own (GEMM8_LDS): A0 A1 A2 B0 B1, or S0 S1 S2.
  static constexpr bool RING = BM == 256;
  static constexpr int N_OBJ = RING ? 5 : 3;
  static constexpr int OBJ = RING ? HALF : STAGE;
  static constexpr int RA = 3, RB = 2;              // ring depths (A, B)

  static FC_DEVICE int off(int row, int c) { return row * 128 + ((c ^ ((row >> 1) & 7)) << 4); }

  // Wave w fills 1 KB blocks (8 rows each) w, w + 8, ... of both operands
  // (an A-then-B stage); with h >= 0 only the blocks w + 8 j with j mod 2 = h.
  static FC_DEVICE void dma(char* stage, __amdgpu_buffer_rsrc_t da, int lda, __amdgpu_buffer_rsrc_t db,
                            int ldb, int m0, int n0, int k0, int wave, int lane, int h = -1) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      // BM 128, half h: A block h and B blocks h, h + 2 (three loads each)
      if (h >= 0 && (j & 1) != h) continue;
      const int blk = wave + 8 * j;
      const int row = blk * 8 + (lane >> 3);
      const int c = (lane & 7) ^ ((row >> 1) & 7);
      if (j < BM / 64)  // BM/8 blocks of A: 4 per wave (BM 256) or 2 (BM 128)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(da, (lds_void_t*)(stage + blk * 1024), 16,
                                                 ((m0 + row) * lda + k0 + c * 8) * 2, 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(db, (lds_void_t*)(stage + HALF_A + blk * 1024), 16,
                                               ((n0 + row) * ldb + k0 + c * 8) * 2, 0, 0, 0);
    }
  }

  // One operand's slice into a ring stage: wave w fills 1 KB blocks (8 rows
  // each) w, w + 8, w + 16, w + 24 (256 rows).
  static FC_DEVICE void dma_op(char* stage, __amdgpu_buffer_rsrc_t d, int ld, int r0, int k0, int wave,
                               int lane) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int blk = wave + 8 * j;
      const int row = blk * 8 + (lane >> 3);
      const int c = (lane & 7) ^ ((row >> 1) & 7);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(d, (lds_void_t*)(stage + blk * 1024), 16,
                                               ((r0 + row) * ld + k0 + c * 8) * 2, 0, 0, 0);
    }
  }

  // fragments of k16 step kk (0..3) of a slice whose A and B parts start at sa, sb
  static FC_DEVICE void frags(const char* sa, const char* sb, int kk, int wm, int wn, int lane,
                              bf16x8_t (&af)[MB], bf16x8_t (&bfr)[NB]) {
    const int lr = lane & 31, c = kk * 2 + (lane >> 5);
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
      af[mb] = as_bf16x8(*(const u32x4_t*)(sa + off(wm * WROWS + mb * 32 + lr, c)));
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
      bfr[nb] = as_bf16x8(*(const u32x4_t*)(sb + off(wn * 128 + nb * 32 + lr, c)));
  }

  // An 8 KB LDS region per wave that no load writes between the end of
  // main_loop() and the next main_loop(), even with the next tile's first
  // slices requested by prologue(): for an epilogue's staging.
  static FC_DEVICE char* epi(char* const (&st)[5], int wave) {
    if constexpr (RING)
      return wave < 4 ? st[2] + wave * 8192 : st[4] + (wave - 4) * 8192;
    else
      return wave < 6 ? st[1] + wave * 8192 : st[2] + (wave - 6) * 8192;
  }

  static FC_DEVICE void mma(const bf16x8_t (&af)[MB], const bf16x8_t (&bfr)[NB], f32x16_t (&acc)[MB][NB]) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) acc[mb][nb] = mfma32x32x16(af[mb], bfr[nb], acc[mb][nb]);
  }

  // Phase boundaries; the scheduling barriers keep MFMAs and memory operations
  // on their own side of them.
  static FC_DEVICE void bar() {
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
  }
  // LDS hand-over: this wave's LDS reads are complete (its direct-to-LDS loads
  // are covered by an explicit vmcnt wait where needed).
  static FC_DEVICE void lds_bar() {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
  }

  // Requests the first slices (the part of run() that may be issued early, e.g.
  // before the previous tile's epilogue): 256-row tiles A(0), B(0), A(1);
  // 128-row tiles slices 0 and 1.
  static FC_DEVICE void prologue(const uint16_t* __restrict__ A, int lda, int M,
                                 const uint16_t* __restrict__ Bm, int ldb, int N, int K, int m0,
                                 int n0, char* const (&st)[5]) {
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const __amdgpu_buffer_rsrc_t da = make_rsrc(A, (uint32_t)M * lda * 2);
    const __amdgpu_buffer_rsrc_t db = make_rsrc(Bm, (uint32_t)N * ldb * 2);
    const __amdgpu_buffer_rsrc_t dz = make_rsrc(A, 0);
    const int KS = K / BK;
    if constexpr (RING) {
      dma_op(st[0], KS > 0 ? da : dz, lda, m0, 0, wave, lane);
      dma_op(st[RA], KS > 0 ? db : dz, ldb, n0, 0, wave, lane);
      dma_op(st[1], KS > 1 ? da : dz, lda, m0, BK, wave, lane);
    } else {
#pragma unroll
      for (int j = 0; j < NST - 1; ++j) {
        const bool more = j < KS;
        dma(st[j], more ? da : dz, lda, more ? db : dz, ldb, m0, n0, j * BK, wave, lane);
      }
    }
  }

  // acc = A[m0 .., 0 .. K) . Bm[n0 .., 0 .. K)^T for the tile; rows past M or N
  // read as 0. K must be a multiple of 64. st: the N_OBJ distinct __shared__
  // arrays of GEMM8_LDS (distinct objects, so the compiler sees that fragment
  // reads of one stage do not depend on loads landing in another and adds no
  // wait of its own). Loads past the last slice go through a zero-range buffer
  // descriptor (no memory access), so every slice issues the same loads and the
  // wait counts are constants. Ends with every load landed and a barrier, so
  // the caller may reuse the stages.
  static FC_DEVICE void run(const uint16_t* __restrict__ A, int lda, int M,
                            const uint16_t* __restrict__ Bm, int ldb, int N, int K, int m0, int n0,
                            char* const (&st)[5], f32x16_t (&acc)[MB][NB]) {
    prologue(A, lda, M, Bm, ldb, N, K, m0, n0, st);
    main_loop<false>(A, lda, M, Bm, ldb, N, K, m0, n0, st, acc);
  }

  // The rest of run() after prologue(). AFTER_OTHER: other vector memory
  // operations were issued after the prologue (a previous tile's epilogue), so
  // the first wait is for everything outstanding.
  template <bool AFTER_OTHER>
  static FC_DEVICE void main_loop(const uint16_t* __restrict__ A, int lda, int M,
                                  const uint16_t* __restrict__ Bm, int ldb, int N, int K, int m0,
                                  int n0, char* const (&st)[5], f32x16_t (&acc)[MB][NB]) {
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = wave >> 1, wn = wave & 1;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[mb][nb][i] = 0.f;
    const __amdgpu_buffer_rsrc_t da = make_rsrc(A, (uint32_t)M * lda * 2);
    const __amdgpu_buffer_rsrc_t db = make_rsrc(Bm, (uint32_t)N * ldb * 2);
    const __amdgpu_buffer_rsrc_t dz = make_rsrc(A, 0);
    const int KS = K / BK;
    bf16x8_t a0[MB], b0[NB], a1[MB], b1[NB];
    if constexpr (RING) {
      // slice s: A in st[s mod 3], B in st[3 + s mod 2]
      if (AFTER_OTHER)
        FC_WAIT_VMCNT(0);
      else
        FC_WAIT_VMCNT(DMA_A);  // A(0) and B(0) landed (for this wave); A(1) may be in flight
      lds_bar();
      if (wm >= 2) bar();  // the second half of the tile rows starts half a period later
      for (int w = 0; w < KS; w += RA * RB) {
#pragma unroll
        for (int u = 0; u < RA * RB; ++u) {
          const int s = w + u;
          if (s < KS) {  // uniform over the workgroup
            const char* ca = st[u % RA];
            const char* cb = st[RA + u % RB];
            // first half-slice; refill: this wave's B blocks of slice s + 1, into the
            // B stage slice s - 1 used (read by both groups before the last barrier)
            dma_op(st[RA + (u + 1) % RB], s + 1 < KS ? db : dz, ldb, n0, (s + 1) * BK, wave, lane);
            frags(ca, cb, 0, wm, wn, lane, a0, b0);
            frags(ca, cb, 1, wm, wn, lane, a1, b1);
            lds_bar();
            mma(a0, b0, acc);
            mma(a1, b1, acc);
            bar();
            // second half-slice; refill: this wave's A blocks of slice s + 2, into the
            // A stage slice s - 1 used
            dma_op(st[(u + 2) % RA], s + 2 < KS ? da : dz, lda, m0, (s + 2) * BK, wave, lane);
            frags(ca, cb, 2, wm, wn, lane, a0, b0);
            frags(ca, cb, 3, wm, wn, lane, a1, b1);
            FC_WAIT_VMCNT(DMA_A);  // all but A(s + 2): B(s + 1) and A(s + 1) landed (this wave)
            lds_bar();
            mma(a0, b0, acc);
            mma(a1, b1, acc);
            bar();
          }
        }
      }
      if (wm < 2) bar();
      FC_WAIT_VMCNT(0);  // the last refills (zero-range) have landed too
      __syncthreads();
    } else {
      if (AFTER_OTHER)
        FC_WAIT_VMCNT(0);
      else
        FC_WAIT_VMCNT((NST - 2) * DMA_N);  // slice 0 landed (for this wave)
      lds_bar();
      if (wm >= 2) bar();  // the second half of the tile rows starts half a period later
      // slice s lives in stage s mod NST and is requested NST - 1 slices ahead; the
      // slice count is padded to a multiple of NST (MFMAs skipped past the end)
      for (int w = 0; w < KS; w += NST) {
#pragma unroll
        for (int q = 0; q < 2 * NST; ++q) {  // half-slices of slices w .. w + NST - 1
          const int j = q >> 1;
          const int ws = w + j;
          char* cur = st[j];
          // memory phase: half of this wave's loads of slice ws + NST - 1 on each
          // half-slice (the 48 KB of a slice take longer on the load path than
          // its MFMAs, so they are spread over all four phases of the slice)
          {
            const int nxt = ws + NST - 1;
            const bool more = nxt < KS;
            dma(st[(j + NST - 1) % NST], more ? da : dz, lda, more ? db : dz, ldb, m0, n0, nxt * BK,
                wave, lane, q & 1);
          }
          frags(cur, cur + HALF_A, 2 * (q & 1), wm, wn, lane, a0, b0);
          frags(cur, cur + HALF_A, 2 * (q & 1) + 1, wm, wn, lane, a1, b1);
          if (q & 1) FC_WAIT_VMCNT((NST - 2) * DMA_N);  // slice ws + 1 landed (for this wave)
          lds_bar();
          // compute phase
          if (ws < KS) {
            mma(a0, b0, acc);
            mma(a1, b1, acc);
          }
          bar();
        }
      }
      if (wm < 2) bar();
      __syncthreads();
    }
  }
};

// The LDS objects of a Gemm8<BM> pipeline in a kernel, as distinct __shared__
// arrays, and the array of their addresses that its functions take.
#define GEMM8_LDS(G, st)                                                                   \
  __shared__ __attribute__((aligned(1024))) char st##_o0[G::OBJ];                           \
  __shared__ __attribute__((aligned(1024))) char st##_o1[G::OBJ];                           \
  __shared__ __attribute__((aligned(1024))) char st##_o2[G::OBJ];                           \
  __shared__ __attribute__((aligned(1024))) char st##_o3[G::N_OBJ > 3 ? G::OBJ : 16];       \
  __shared__ __attribute__((aligned(1024))) char st##_o4[G::N_OBJ > 4 ? G::OBJ : 16];       \
  char* const st[5] = {st##_o0, st##_o1, st##_o2, st##_o3, st##_o4}

// Tile height of Gemm8 for an M-row product with n_tiles_n 256-wide column tiles:
// the one with fewer rounds of workgroups over the device's CUs, weighting a
// 128-row tile (three stages) at 0.62 of a 256-row one (two stages, before the
// A and B rings, which made 256-row tiles 8 % faster): measured
// 0.58 to 0.63 for M from 1024 to 8192 with 16 or 48 column tiles.
#ifndef FC_GEMM8_FORCE_BM
inline int gemm8_pick_bm(int M, int n_tiles_n) {
  const int n_cu = fc_num_cus();
  const long t256 = (long)((M + 255) / 256) * n_tiles_n, t128 = (long)((M + 127) / 128) * n_tiles_n;
  const long r256 = (t256 + n_cu - 1) / n_cu, r128 = (t128 + n_cu - 1) / n_cu;
  return r128 * 62 < r256 * 100 ? 128 : 256;
}
#else
inline int gemm8_pick_bm(int, int) { return FC_GEMM8_FORCE_BM; }
#endif
