// LM head with the Flash-Verify accept test fused into its epilogue: logits =
// hidden . W^T over the whole vocabulary, reduced per row to the argmax (lowest
// token id among the maxima) and the confidence (largest softmax probability),
// then the two-view accept test; the [R, vocab] logits never reach memory.
//
// Flash-Verify accepts the draft and [MASK] predictions that meet the
// confidence threshold (infernews post "Flash-dLLM 讓擴散式語言模型解碼更快、
// 更省記憶體", paragraph 3; threshold 0.9 in the README quote of the zhichai.net
// forum post, section 4); the predictions come from the model's logits.
//
// The GEMM is the projection's tile pipeline (gemm_tile.hpp, Gemm8 with
// 256-row tiles, persistent over the tiles; each XCD takes whole 256-column
// blocks of W and runs every row tile of a block before the next, so W is
// streamed from memory once). Epilogue per tile: each wave holds 64 rows x
// 128 vocabulary columns as fp32 accumulators; per row it reduces them to
// (max m, lowest column holding m, sum of exp(x - m)) across its 32 lanes
// with butterfly exchanges and writes that partial. A second kernel merges the
// 2 * vocab / 256 partials of a row in a fixed order (deterministic),
// computes conf = 1 / sum and applies the accept rule of fv_verify_accept.
#include "gemm_tile.hpp"

namespace {

constexpr float LOG2E_L = 1.4426950408889634f;
// column blocks of W an XCD's workgroups share at one time (tile order below):
// at 4366 rows x 126464 columns, 1, 2, 4, 8, 16 and 32 give 4237-4324, 4188,
// 4108, 3998-4190, 4386 and 5175 us in one A/B run
constexpr int LMHEAD_COL_GROUP = 8;

struct Part {
  float m, s;
  int idx;
};

__global__ __launch_bounds__(Gemm8<256>::THREADS, 1) void lmhead_partials(
    const uint16_t* __restrict__ hidden, int M, const uint16_t* __restrict__ w, int d,
    int n_tiles_n, int n_tiles, int grp, Part* __restrict__ part) {
  using G = Gemm8<256>;
  GEMM8_LDS(G, sts);
  const int t = threadIdx.x, lane = t & 63, lr = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int N = n_tiles_n * G::BN;
  const int n_part = 2 * n_tiles_n;
  // Tile order. W (vocab x d) is far larger than the Infinity Cache, so each
  // 256-column block of it must be streamed once and then serve every row
  // tile from L2: workgroup g (placed on XCD g mod 8) walks the column blocks
  // nt = g mod 8, + 8, ... of that XCD in groups of `grp` blocks, all row tiles
  // of one group before the next, the group's blocks fastest: the tiles an
  // XCD runs at one time then share grp blocks of W and few row blocks of the
  // hidden states. Any placement gives the same result.
  const int n_tiles_m = n_tiles / n_tiles_n;
  const int xcd = blockIdx.x & 7, per_xcd = gridDim.x >> 3;   // gridDim.x is a multiple of 8
  const int n_blk = (n_tiles_n - xcd + 7) >> 3;                  // column blocks of this XCD
  const int my_tiles = n_blk * n_tiles_m;
  int j = blockIdx.x >> 3;
  if (j >= my_tiles) return;
  const int per_grp = grp * n_tiles_m;
  auto coords = [&](int jj, int& mt, int& nt) {
    const int g = jj / per_grp, r = jj - g * per_grp;
    const int gsz = min(grp, n_blk - g * grp);   // the last group may be smaller
    mt = r / gsz;
    nt = xcd + 8 * (g * grp + r % gsz);
  };
  int mt, nt;
  coords(j, mt, nt);
  G::prologue(hidden, d, M, w, d, N, d, mt * G::BM, nt * G::BN, sts);
  for (;;) {
    const int m0 = mt * G::BM, n0 = nt * G::BN;
    f32x16_t acc[G::MB][G::NB];
    G::template main_loop<true>(hidden, d, M, w, d, N, d, m0, n0, sts, acc);
    const int jn = j + per_xcd;
    int mt_n = 0, nt_n = 0;
    if (jn < my_tiles) {
      coords(jn, mt_n, nt_n);
      G::prologue(hidden, d, M, w, d, N, d, mt_n * G::BM, nt_n * G::BN, sts);
    }
    const int col0 = n0 + wn * 128;
#pragma unroll
    for (int mb = 0; mb < G::MB; ++mb) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        // this lane's 4 columns of the row (col0 + nb * 32 + lr): max, lowest column
        float m = acc[mb][0][i];
        int idx = col0 + lr;
#pragma unroll
        for (int nb = 1; nb < G::NB; ++nb)
          if (acc[mb][nb][i] > m) {
            m = acc[mb][nb][i];
            idx = col0 + nb * 32 + lr;
          }
        // across the 32 lanes of the row group (xor offsets below 32 stay in it)
#pragma unroll
        for (int off = 16; off >= 1; off >>= 1) {
          const float om = __shfl_xor(m, off);
          const int oi = __shfl_xor(idx, off);
          if (om > m || (om == m && oi < idx)) {
            m = om;
            idx = oi;
          }
        }
        const float ml = m * LOG2E_L;
        float s = 0.f;
#pragma unroll
        for (int nb = 0; nb < G::NB; ++nb) s += __builtin_amdgcn_exp2f(fmaf(acc[mb][nb][i], LOG2E_L, -ml));
#pragma unroll
        for (int off = 16; off >= 1; off >>= 1) s += __shfl_xor(s, off);
        const int row = m0 + wm * G::WROWS + acc_row(mb, i, lane);
        if (lr == 0 && row < M) part[(size_t)row * n_part + nt * 2 + wn] = Part{m, s, idx};
      }
    }
    j = jn;
    if (j >= my_tiles) break;
    mt = mt_n;
    nt = nt_n;
  }
}

FC_DEVICE int seq_of(const int32_t* __restrict__ cu, int B, int x) {
  int lo = 0, hi = B;  // cu[lo] <= x < cu[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (cu[mid] <= x) lo = mid; else hi = mid;
  }
  return lo;
}

// One workgroup of 256 threads per row: thread j merges partials j, j + 256,
// ... in order, then a fixed tree combines the threads.
__global__ __launch_bounds__(256) void lmhead_finish(const Part* __restrict__ part, int n_part,
                                                     const int32_t* __restrict__ cu_p, int B,
                                                     const int32_t* __restrict__ draft, float tau,
                                                     int32_t* __restrict__ argmax,
                                                     float* __restrict__ conf,
                                                     uint8_t* __restrict__ accept_row) {
  __shared__ float s_m[4], s_s[4];
  __shared__ int s_i[4];
  const int r = blockIdx.x, t = threadIdx.x;
  float m = -INFINITY, s = 0.f;
  int idx = 0x7FFFFFFF;
  auto merge = [](float& m, float& s, int& idx, float om, float os, int oi) {
    if (om == -INFINITY) return;  // an empty partial (a thread or wave without partials)
    if (om > m) {
      s = s * __builtin_amdgcn_exp2f((m - om) * LOG2E_L) + os;
      m = om;
      idx = oi;
    } else {
      s += os * __builtin_amdgcn_exp2f((om - m) * LOG2E_L);
      if (om == m && oi < idx) idx = oi;
    }
  };
  for (int j = t; j < n_part; j += 256) {
    const Part p = part[(size_t)r * n_part + j];
    merge(m, s, idx, p.m, p.s, p.idx);
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const float om = __shfl_xor(m, off), os = __shfl_xor(s, off);
    const int oi = __shfl_xor(idx, off);
    merge(m, s, idx, om, os, oi);
  }
  if ((t & 63) == 0) {
    s_m[t >> 6] = m;
    s_s[t >> 6] = s;
    s_i[t >> 6] = idx;
  }
  __syncthreads();
  if (t == 0) {
    m = s_m[0];
    s = s_s[0];
    idx = s_i[0];
    for (int w = 1; w < 4; ++w) merge(m, s, idx, s_m[w], s_s[w], s_i[w]);
    const float c = 1.f / s;
    const int b = seq_of(cu_p, B, r >> 1);
    const int p0 = cu_p[b], n = cu_p[b + 1] - p0;
    const int local = r - 2 * p0;
    const int i = local >= n ? local - n : local;
    argmax[r] = idx;
    conf[r] = c;
    accept_row[r] = (uint8_t)(idx == draft[p0 + i] && c >= tau);
  }
}

__global__ void lmhead_positions(const uint8_t* __restrict__ accept_row,
                                 const int32_t* __restrict__ cu_p, int B, int n_pos,
                                 uint8_t* __restrict__ accept_pos) {
  const int p = blockIdx.x * blockDim.x + threadIdx.x;
  if (p >= n_pos) return;
  const int b = seq_of(cu_p, B, p);
  const int p0 = cu_p[b], n = cu_p[b + 1] - p0;
  const int i = p - p0;
  accept_pos[p] = accept_row[2 * p0 + i] & accept_row[2 * p0 + n + i];
}

}  // namespace

extern "C" size_t fv_lmhead_workspace_size(int32_t R, int32_t vocab) {
  if (R <= 0 || vocab <= 0) return 0;
  const size_t n_part = 2 * (((size_t)vocab + 255) / 256);
  return (size_t)R * n_part * sizeof(Part);
}

extern "C" fc_status_t fv_lmhead_verify_accept(const void* hidden, const void* w_lm,
                                               int32_t d_model, int32_t vocab,
                                               const int32_t* cu_positions, int32_t B, int32_t R,
                                               const int32_t* draft_tokens, float tau,
                                               void* workspace, size_t workspace_bytes,
                                               int32_t* argmax, float* conf, uint8_t* accept_row,
                                               uint8_t* accept_pos, fc_stream_t stream) {
  fc_clear_error();
  FC_REQUIRE(B >= 1 && vocab >= 1 && d_model >= 1 && R >= 0 && (R % 2) == 0, FC_ERR_INVALID_VALUE,
             "fv_lmhead_verify_accept: bad sizes B=%d vocab=%d d_model=%d R=%d (R even)", B, vocab,
             d_model, R);
  FC_REQUIRE(tau > 0.f && tau <= 1.f, FC_ERR_INVALID_VALUE,
             "fv_lmhead_verify_accept: tau=%g must be in (0, 1]", (double)tau);
  FC_REQUIRE(vocab % 256 == 0 && d_model % 64 == 0, FC_ERR_UNSUPPORTED,
             "fv_lmhead_verify_accept: needs vocab %% 256 == 0 and d_model %% 64 == 0 (got %d, %d)",
             vocab, d_model);
  FC_REQUIRE((int64_t)R * d_model * 2 < (1ll << 31) && (int64_t)vocab * d_model * 2 < (1ll << 31),
             FC_ERR_UNSUPPORTED, "fv_lmhead_verify_accept: operands too large");
  FC_REQUIRE(cu_positions && (R == 0 || (hidden && w_lm && draft_tokens && argmax && conf &&
                                         accept_row)),
             FC_ERR_INVALID_VALUE, "fv_lmhead_verify_accept: NULL required pointer");
  if (R == 0) return FC_OK;
  FC_REQUIRE(workspace && workspace_bytes >= fv_lmhead_workspace_size(R, vocab), FC_ERR_WORKSPACE,
             "fv_lmhead_verify_accept: workspace of %zu bytes required",
             fv_lmhead_workspace_size(R, vocab));
  FC_REQUIRE((((uintptr_t)hidden | (uintptr_t)w_lm | (uintptr_t)workspace) & 15) == 0,
             FC_ERR_INVALID_VALUE, "fv_lmhead_verify_accept: pointers must be 16-byte aligned");
  hipStream_t st = (hipStream_t)stream;
  if (fc_debug_enabled()) {
    const fc_status_t s = fc_debug_check_offsets(cu_positions, B, R / 2, "cu_positions",
                                                 "fv_lmhead_verify_accept (FC_DEBUG)", st);
    if (s != FC_OK) return s;
  }
  const int n_tiles_n = vocab / 256;
  const int n_tiles = ((R + 255) / 256) * n_tiles_n;
  // persistent: one workgroup per CU (a multiple of 8, the XCD count), each
  // walking its XCD's column blocks; workgroups beyond an XCD's tiles exit
  const int grid = fc_num_cus() >= 8 ? fc_num_cus() / 8 * 8 : 8;
  hipLaunchKernelGGL(lmhead_partials, dim3(grid), dim3(Gemm8<256>::THREADS), 0, st,
                     (const uint16_t*)hidden, R, (const uint16_t*)w_lm, d_model, n_tiles_n, n_tiles,
                     LMHEAD_COL_GROUP, (Part*)workspace);
  fc_status_t s = fc_check_launch("fv_lmhead_verify_accept");
  if (s != FC_OK) return s;
  hipLaunchKernelGGL(lmhead_finish, dim3(R), dim3(256), 0, st, (const Part*)workspace,
                     2 * n_tiles_n, cu_positions, B, draft_tokens, tau, argmax, conf, accept_row);
  s = fc_check_launch("fv_lmhead_verify_accept");
  if (s != FC_OK || !accept_pos) return s;
  const int n_pos = R / 2;
  hipLaunchKernelGGL(lmhead_positions, dim3((n_pos + 255) / 256), dim3(256), 0, st, accept_row,
                     cu_positions, B, n_pos, accept_pos);
  return fc_check_launch("fv_lmhead_verify_accept");
}
