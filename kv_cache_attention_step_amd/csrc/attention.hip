// Bidirectional varlen attention over the paged KV cache with the per-key
// attention importance fused in.
//
// Method: each step the fixed-size query of a sequence attends bidirectionally
// (no mask) to the sequence's full KV cache, and the tracked positions for the
// next step are chosen by attention importance (signal-papers page on arXiv
// 2609.26796, Fig. 2); sequences of different query lengths share one
// block-scheduled launch (infernews post "Flash-dLLM 讓擴散式語言模型解碼更快、
// 更省記憶體", paragraph 2).
//
// gfx950 design (bf16, D = 128). One workgroup of 4 waves serves one
// (sequence, head) and up to 128 query rows (32 per wave), so every K/V byte of
// that head is fetched from HBM once and shared by all query rows through LDS.
// Per 64-key tile:
//   * K tile [64 keys][128] and V tile, transposed to V^T [128][64], are staged in
//     LDS (double buffered; the next tile's global loads are in flight while the
//     current one is consumed).
//   * S^T = K Q^T with v_mfma_f32_32x32x16_bf16: the accumulator of a 32x32
//     block gives each lane one query (lane % 32) and 16 keys, so row statistics
//     need only one cross-half exchange, and the probabilities are already in the
//     B-operand layout of O^T += V^T P^T (the 16 keys of a lane pair up with the
//     MFMA k index through a fixed permutation, applied identically to V^T).
//   * Importance needs the column sums of the *normalised* P, whose row
//     normaliser is known only after all keys were seen. The kernel therefore
//     runs two passes over the keys: pass 1 (K only) computes each row's max and
//     normaliser; pass 2 recomputes S bit-identically, forms exact P, accumulates
//     O and reduces P over the query rows: a 5-step transpose-reduce across the
//     32 lanes of each half-wave leaves one key sum per lane, and the four waves
//     are summed in fixed order through LDS. No float atomics: importance is
//     deterministic. The second K pass mostly hits L2/MALL (the same head's keys
//     were just read).
//   * Without importance (verify pass) a single online-softmax pass is used.
#include "fc_common.hpp"

#include <math.h>

namespace {

constexpr int AD = 128;                 // head dim
constexpr int AKT = 64;                 // keys per tile
constexpr int AROWS = 128;              // query rows per workgroup pass
constexpr int K_STRIDE = AD * 2 + 16;   // bytes per key row of the K tile
constexpr int V_STRIDE = AKT * 2 + 8;   // bytes per dim row of the V^T tile
constexpr int K_TILE = AKT * K_STRIDE;
constexpr int V_TILE = AD * V_STRIDE;
constexpr int A_STAGE = K_TILE + V_TILE;
constexpr int A_RED = 2 * 4 * AKT * 4;  // double-buffered [wave][key] fp32 partial sums
constexpr int A_LDS = 2 * A_STAGE + A_RED;
constexpr float LOG2E = 1.4426950408889634f;

struct AttnArgs {
  const uint16_t* q;
  const uint16_t* kc;
  const uint16_t* vc;
  const int32_t* block_table;
  const int32_t* cu_q;
  const int32_t* cu_k;
  uint16_t* out;
  float* imp;
  int maxp, log2ps, B, H, T_k, n_rt, accumulate;
  float scale_log2;  // softmax_scale * log2(e)
};

// ---- tile loads ----------------------------------------------------------
// K: thread t loads 16-byte chunk (t & 15) of keys (t >> 4) + 16 j, j < 4.
FC_DEVICE void load_k(const AttnArgs& a, const int32_t* bt, int h, int tile, int L,
                      u32x4_t (&r)[4]) {
  const int t = threadIdx.x;
  const int psm = (1 << a.log2ps) - 1;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int key = tile * AKT + (t >> 4) + 16 * j;
    if (key < L) {
      const int page = bt[key >> a.log2ps];
      const size_t off = (((size_t)page * a.H + h) * (psm + 1) + (key & psm)) * AD + (t & 15) * 8;
      r[j] = *(const u32x4_t*)(a.kc + off);
    } else {
      r[j] = u32x4_t{0, 0, 0, 0};
    }
  }
}
FC_DEVICE void store_k(char* ks, const u32x4_t (&r)[4]) {
  const int t = threadIdx.x;
#pragma unroll
  for (int j = 0; j < 4; ++j) *(u32x4_t*)(ks + ((t >> 4) + 16 * j) * K_STRIDE + (t & 15) * 16) = r[j];
}
// V: thread t loads keys 4 (t & 15) .. +3, dims 8 (t >> 4) .. +7, and writes them
// transposed (4 keys of one dim = 8 bytes) into V^T.
FC_DEVICE void load_v(const AttnArgs& a, const int32_t* bt, int h, int tile, int L,
                      u32x4_t (&r)[4]) {
  const int t = threadIdx.x;
  const int psm = (1 << a.log2ps) - 1;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int key = tile * AKT + 4 * (t & 15) + j;
    if (key < L) {
      const int page = bt[key >> a.log2ps];
      const size_t off = (((size_t)page * a.H + h) * (psm + 1) + (key & psm)) * AD + (t >> 4) * 8;
      r[j] = *(const u32x4_t*)(a.vc + off);
    } else {
      r[j] = u32x4_t{0, 0, 0, 0};
    }
  }
}
FC_DEVICE void store_v(char* vs, const u32x4_t (&r)[4]) {
  const int t = threadIdx.x;
  const int key0 = 4 * (t & 15);
  const int d0 = 8 * (t >> 4);
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    // r[j][p] holds dims (d0 + 2p) in its low half and (d0 + 2p + 1) in its high half
    const uint32_t w0 = r[0][p], w1 = r[1][p], w2 = r[2][p], w3 = r[3][p];
    u32x2_t lo, hi;
    lo[0] = (w0 & 0xFFFFu) | (w1 << 16);
    lo[1] = (w2 & 0xFFFFu) | (w3 << 16);
    hi[0] = (w0 >> 16) | (w1 & 0xFFFF0000u);
    hi[1] = (w2 >> 16) | (w3 & 0xFFFF0000u);
    *(u32x2_t*)(vs + (d0 + 2 * p) * V_STRIDE + key0 * 2) = lo;
    *(u32x2_t*)(vs + (d0 + 2 * p + 1) * V_STRIDE + key0 * 2) = hi;
  }
}

// ---- MFMA pieces -----------------------------------------------------------
// S^T block kb (keys kb*32 .. +31 of the tile) for this wave's 32 queries.
FC_DEVICE f32x16_t s_block(const char* ks, int kb, const bf16x8_t (&qf)[8], int lane) {
  f32x16_t s = {};
  const char* row = ks + (kb * 32 + (lane & 31)) * K_STRIDE + (lane >> 5) * 16;
#pragma unroll
  for (int kc = 0; kc < 8; ++kc) s = mfma32x32x16(as_bf16x8(*(const u32x4_t*)(row + kc * 32)), qf[kc], s);
  return s;
}

// key (within the tile) of register i of S^T block kb in this lane
FC_DEVICE int s_key(int kb, int i, int lane) { return kb * 32 + (i >> 2) * 8 + (lane >> 5) * 4 + (i & 3); }

// O^T += V^T P^T for the 16 keys of chunk c of block kb; p holds block kb's
// probabilities (16 registers).
FC_DEVICE void pv_chunk(const char* vs, int kb, int c, const f32x16_t& p, f32x16_t (&o)[4],
                        int lane) {
  u32x4_t pb;
#pragma unroll
  for (int w = 0; w < 4; ++w) pb[w] = pack_bf16x2(p[8 * c + 2 * w], p[8 * c + 2 * w + 1]);
  const bf16x8_t bop = as_bf16x8(pb);
  const int kbase = kb * 32 + c * 16 + (lane >> 5) * 4;
#pragma unroll
  for (int db = 0; db < 4; ++db) {
    const char* row = vs + (db * 32 + (lane & 31)) * V_STRIDE + kbase * 2;
    u32x4_t av;
    const u32x2_t x0 = *(const u32x2_t*)row;
    const u32x2_t x1 = *(const u32x2_t*)(row + 16);
    av[0] = x0[0]; av[1] = x0[1]; av[2] = x1[0]; av[3] = x1[1];
    o[db] = mfma32x32x16(as_bf16x8(av), bop, o[db]);
  }
}

FC_DEVICE void load_q(const AttnArgs& a, int q0, int row, int Q, int h, bf16x8_t (&qf)[8]) {
  const int lane = threadIdx.x & 63;
  if (row < Q) {
    const uint16_t* src = a.q + ((size_t)(q0 + row) * a.H + h) * AD + (lane >> 5) * 8;
#pragma unroll
    for (int kc = 0; kc < 8; ++kc) qf[kc] = as_bf16x8(*(const u32x4_t*)(src + kc * 16));
  } else {
#pragma unroll
    for (int kc = 0; kc < 8; ++kc) qf[kc] = as_bf16x8(u32x4_t{0, 0, 0, 0});
  }
}

FC_DEVICE void store_o(const AttnArgs& a, int q0, int row, int Q, int h, const f32x16_t (&o)[4],
                       float scale) {
  if (row >= Q) return;
  const int lane = threadIdx.x & 63;
  uint16_t* dst = a.out + ((size_t)(q0 + row) * a.H + h) * AD + (lane >> 5) * 4;
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      u32x2_t w;
      w[0] = pack_bf16x2(o[db][4 * g] * scale, o[db][4 * g + 1] * scale);
      w[1] = pack_bf16x2(o[db][4 * g + 2] * scale, o[db][4 * g + 3] * scale);
      *(u32x2_t*)(dst + db * 32 + g * 8) = w;
    }
}

// Sum over the 32 lanes of each half-wave of the 16 values a lane holds;
// afterwards lanes l and l^1 both hold the sum of value index (l >> 1) & 15.
FC_DEVICE float transpose_reduce16(f32x16_t& v, int lane) {
#pragma unroll
  for (int m = 8; m >= 1; m >>= 1) {
    const int lm = m * 2;  // lane bit that decides which half of the values is kept
    const bool up = (lane & lm) != 0;
#pragma unroll
    for (int j = 0; j < m; ++j) {
      const float send = up ? v[j] : v[j + m];
      const float keep = up ? v[j + m] : v[j];
      v[j] = keep + __shfl_xor(send, lm);
    }
  }
  return v[0] + __shfl_xor(v[0], 1);
}

// ---- kernels -------------------------------------------------------------------
template <bool WITH_IMP>
__global__ __launch_bounds__(256, 2) void attn_bf16_d128(AttnArgs a) {
  __shared__ __attribute__((aligned(16))) char lds[A_LDS];
  float* red = (float*)(lds + 2 * A_STAGE);

  int item = blockIdx.x;
  int rt_begin, rt_end;
  int b, h;
  if (WITH_IMP) {
    b = item / a.H;
    h = item % a.H;
    rt_begin = 0;
    rt_end = a.n_rt;
  } else {
    const int rt = item % a.n_rt;
    item /= a.n_rt;
    b = item / a.H;
    h = item % a.H;
    rt_begin = rt;
    rt_end = rt + 1;
  }
  const int q0 = a.cu_q[b], Q = a.cu_q[b + 1] - q0;
  const int k0 = a.cu_k[b], L = a.cu_k[b + 1] - k0;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int32_t* bt = a.block_table + (size_t)b * a.maxp;
  const int n_tiles = (L + AKT - 1) / AKT;

  if (WITH_IMP && Q == 0 && !a.accumulate) {  // no query rows: column sums are 0
    for (int key = t; key < L; key += blockDim.x) a.imp[(size_t)h * a.T_k + k0 + key] = 0.f;
    return;
  }
  for (int rt = rt_begin; rt < rt_end; ++rt) {
    if (rt * AROWS >= Q) break;
    const int row = rt * AROWS + wave * 32 + (lane & 31);
    const bool row_ok = row < Q;
    if (L == 0) {  // no keys: output 0
      const f32x16_t z[4] = {};
      store_o(a, q0, row, Q, h, z, 1.f);
      continue;
    }
    bf16x8_t qf[8];
    load_q(a, q0, row, Q, h, qf);
    f32x16_t o[4] = {};
    u32x4_t rk[4], rv[4];

    if (WITH_IMP) {
      // ---------------- pass 1: row max and normaliser ----------------
      float m = -INFINITY, l = 0.f;
      load_k(a, bt, h, 0, L, rk);
      store_k(lds, rk);
      __syncthreads();
      for (int tile = 0; tile < n_tiles; ++tile) {
        const bool more = tile + 1 < n_tiles;
        if (more) load_k(a, bt, h, tile + 1, L, rk);
        const char* ks = lds + (tile & 1) * A_STAGE;
        float x[32];
        float tmax = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const f32x16_t s = s_block(ks, kb, qf, lane);
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int key = tile * AKT + s_key(kb, i, lane);
            const float v = key < L ? s[i] * a.scale_log2 : -INFINITY;
            x[kb * 16 + i] = v;
            tmax = fmaxf(tmax, v);
          }
        }
        const float mn = fmaxf(m, tmax);
        const float mref = mn == -INFINITY ? 0.f : mn;  // this lane has seen no key yet
        float sum = 0.f;
#pragma unroll
        for (int j = 0; j < 32; ++j) sum += exp2f(x[j] - mref);
        l = (m == -INFINITY ? 0.f : l * exp2f(m - mn)) + sum;
        m = mn;
        if (more) store_k(lds + ((tile + 1) & 1) * A_STAGE, rk);
        __syncthreads();
      }
      const float mo = __shfl_xor(m, 32), lo = __shfl_xor(l, 32);
      const float mf = fmaxf(m, mo);
      const float lf = (m == -INFINITY ? 0.f : l * exp2f(m - mf)) +
                       (mo == -INFINITY ? 0.f : lo * exp2f(mo - mf));
      const float inv_l = row_ok ? 1.f / lf : 0.f;

      // ---------------- pass 2: P, O += P V, importance ----------------
      load_k(a, bt, h, 0, L, rk);
      load_v(a, bt, h, 0, L, rv);
      store_k(lds, rk);
      store_v(lds + K_TILE, rv);
      __syncthreads();
      for (int tile = 0; tile < n_tiles; ++tile) {
        const bool more = tile + 1 < n_tiles;
        if (more) {
          load_k(a, bt, h, tile + 1, L, rk);
          load_v(a, bt, h, tile + 1, L, rv);
        }
        const char* ks = lds + (tile & 1) * A_STAGE;
        const char* vs = ks + K_TILE;
        float* rb = red + (tile & 1) * 4 * AKT;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          f32x16_t s = s_block(ks, kb, qf, lane);
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int key = tile * AKT + s_key(kb, i, lane);
            s[i] = key < L ? exp2f(s[i] * a.scale_log2 - mf) * inv_l : 0.f;
          }
          pv_chunk(vs, kb, 0, s, o, lane);
          pv_chunk(vs, kb, 1, s, o, lane);
          // column sums over this wave's 32 query rows: lanes l and l^1 end with
          // the sum of register index (l >> 1) & 15
          const float colsum = transpose_reduce16(s, lane);
          if ((lane & 1) == 0) {
            const int r = (lane >> 1) & 15;
            rb[wave * AKT + s_key(kb, r, lane)] = colsum;
          }
        }
        if (more) {
          store_k(lds + ((tile + 1) & 1) * A_STAGE, rk);
          store_v(lds + ((tile + 1) & 1) * A_STAGE + K_TILE, rv);
        }
        __syncthreads();
        if (t < AKT) {
          const int key = tile * AKT + t;
          if (key < L) {
            const float v = rb[t] + rb[AKT + t] + rb[2 * AKT + t] + rb[3 * AKT + t];
            float* dst = a.imp + (size_t)h * a.T_k + k0 + key;
            *dst = (a.accumulate || rt > 0) ? *dst + v : v;
          }
        }
      }
      store_o(a, q0, row, Q, h, o, 1.f);
      __syncthreads();  // LDS reuse by the next row tile
    } else {
      // ---------------- single pass, online softmax ----------------
      float m = -INFINITY, l = 0.f;
      load_k(a, bt, h, 0, L, rk);
      load_v(a, bt, h, 0, L, rv);
      store_k(lds, rk);
      store_v(lds + K_TILE, rv);
      __syncthreads();
      for (int tile = 0; tile < n_tiles; ++tile) {
        const bool more = tile + 1 < n_tiles;
        if (more) {
          load_k(a, bt, h, tile + 1, L, rk);
          load_v(a, bt, h, tile + 1, L, rv);
        }
        const char* ks = lds + (tile & 1) * A_STAGE;
        const char* vs = ks + K_TILE;
        f32x16_t s[2];
        float tmax = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          s[kb] = s_block(ks, kb, qf, lane);
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int key = tile * AKT + s_key(kb, i, lane);
            const float v = key < L ? s[kb][i] * a.scale_log2 : -INFINITY;
            s[kb][i] = v;
            tmax = fmaxf(tmax, v);
          }
        }
        tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
        const float mn = fmaxf(m, tmax);
        const float alpha = m == -INFINITY ? 0.f : exp2f(m - mn);
        float sum = 0.f;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const float p = exp2f(s[kb][i] - mn);
            s[kb][i] = p;
            sum += p;
          }
        l = l * alpha + sum;
        m = mn;
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
          for (int i = 0; i < 16; ++i) o[db][i] *= alpha;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          pv_chunk(vs, kb, 0, s[kb], o, lane);
          pv_chunk(vs, kb, 1, s[kb], o, lane);
        }
        if (more) {
          store_k(lds + ((tile + 1) & 1) * A_STAGE, rk);
          store_v(lds + ((tile + 1) & 1) * A_STAGE + K_TILE, rv);
        }
        __syncthreads();
      }
      const float lt = l + __shfl_xor(l, 32);
      store_o(a, q0, row, Q, h, o, 1.f / lt);
      __syncthreads();
    }
  }
}

// ---- fp32 path (small models): exact two-pass softmax, one thread per query row ----
constexpr int F_ROWS = 64, F_KT = 32;

__global__ __launch_bounds__(64) void attn_f32(const float* __restrict__ q,
                                               const float* __restrict__ kc,
                                               const float* __restrict__ vc,
                                               const int32_t* __restrict__ block_table, int maxp,
                                               int log2ps, const int32_t* __restrict__ cu_q,
                                               const int32_t* __restrict__ cu_k, int H, int D,
                                               float scale, float* __restrict__ out,
                                               float* __restrict__ imp, int T_k, int accumulate) {
  extern __shared__ float fl[];
  float* ks = fl;                       // [F_KT][D]
  float* vs = ks + F_KT * D;            // [F_KT][D]
  float* ps = vs + F_KT * D;            // [F_ROWS][F_KT]
  const int b = blockIdx.x / H, h = blockIdx.x % H;
  const int q0 = cu_q[b], Q = cu_q[b + 1] - q0;
  const int k0 = cu_k[b], L = cu_k[b + 1] - k0;
  const int t = threadIdx.x;
  const int psm = (1 << log2ps) - 1;
  const int32_t* bt = block_table + (size_t)b * maxp;
  float qr[128], o[128];
  if (imp && Q == 0 && !accumulate) {
    for (int key = t; key < L; key += blockDim.x) imp[(size_t)h * T_k + k0 + key] = 0.f;
    return;
  }
  for (int rt = 0; rt * F_ROWS < Q; ++rt) {
    const int row = rt * F_ROWS + t;
    const bool ok = row < Q;
    for (int e = 0; e < D; ++e) {
      qr[e] = ok ? q[((size_t)(q0 + row) * H + h) * D + e] : 0.f;
      o[e] = 0.f;
    }
    float m = -INFINITY, l = 0.f;
    for (int pass = 0; pass < 2; ++pass) {
      for (int k_base = 0; k_base < L; k_base += F_KT) {
        __syncthreads();
        for (int idx = t; idx < F_KT * D; idx += blockDim.x) {
          const int j = idx / D, e = idx % D;
          const int key = k_base + j;
          float kv = 0.f, vv = 0.f;
          if (key < L) {
            const size_t off =
                (((size_t)bt[key >> log2ps] * H + h) * (psm + 1) + (key & psm)) * D + e;
            kv = kc[off];
            vv = vc[off];
          }
          ks[idx] = kv;
          vs[idx] = vv;
        }
        __syncthreads();
        const int nk = min(F_KT, L - k_base);
        for (int j = 0; j < F_KT; ++j) {
          float p = 0.f;
          if (j < nk) {
            float s = 0.f;
            for (int e = 0; e < D; ++e) s = fmaf(qr[e], ks[j * D + e], s);
            s *= scale;
            if (pass == 0) {
              const float mn = fmaxf(m, s);
              l = (m == -INFINITY ? 0.f : l * expf(m - mn)) + expf(s - mn);
              m = mn;
            } else {
              p = ok ? expf(s - m) / l : 0.f;
              for (int e = 0; e < D; ++e) o[e] = fmaf(p, vs[j * D + e], o[e]);
            }
          }
          if (pass == 1) ps[t * F_KT + j] = p;
        }
        if (pass == 1 && imp) {
          __syncthreads();
          if (t < nk) {
            float v = 0.f;
            for (int r = 0; r < F_ROWS; ++r) v += ps[r * F_KT + t];
            float* dst = imp + (size_t)h * T_k + k0 + k_base + t;
            *dst = (accumulate || rt > 0) ? *dst + v : v;
          }
        }
      }
    }
    if (ok)
      for (int e = 0; e < D; ++e) out[((size_t)(q0 + row) * H + h) * D + e] = o[e];
  }
}

}  // namespace

extern "C" size_t fc_attention_workspace_size(int32_t B, int32_t T_q, int32_t T_k, int32_t n_heads,
                                              int32_t head_dim, int32_t with_importance) {
  (void)B; (void)T_q; (void)T_k; (void)n_heads; (void)head_dim; (void)with_importance;
  return 0;
}

extern "C" fc_status_t fc_varlen_bidir_attention(
    const void* q, const void* k_cache, const void* v_cache, const int32_t* block_table,
    int32_t max_pages_per_seq, int32_t page_size, const int32_t* cu_seqlens_q,
    const int32_t* cu_seqlens_k, int32_t B, int32_t max_seqlen_q, int32_t T_k, int32_t n_heads,
    int32_t head_dim, float softmax_scale, void* out, float* importance, int32_t accumulate,
    void* workspace, size_t workspace_bytes, int32_t dtype, fc_stream_t stream) {
  fc_clear_error();
  (void)workspace;
  FC_REQUIRE(B >= 1 && n_heads >= 1 && max_seqlen_q >= 0 && T_k >= 0, FC_ERR_INVALID_VALUE,
             "fc_varlen_bidir_attention: bad sizes B=%d n_heads=%d max_seqlen_q=%d T_k=%d", B,
             n_heads, max_seqlen_q, T_k);
  FC_REQUIRE(dtype == FC_DTYPE_BF16 || dtype == FC_DTYPE_F32, FC_ERR_INVALID_VALUE,
             "fc_varlen_bidir_attention: unknown dtype %d", dtype);
  FC_REQUIRE(q && k_cache && v_cache && block_table && cu_seqlens_q && cu_seqlens_k && out,
             FC_ERR_INVALID_VALUE, "fc_varlen_bidir_attention: NULL required pointer");
  FC_REQUIRE(fc_is_pow2(page_size) && page_size <= 256 && max_pages_per_seq >= 1,
             FC_ERR_INVALID_VALUE,
             "fc_varlen_bidir_attention: page_size=%d must be a power of two <= 256", page_size);
  FC_REQUIRE(softmax_scale > 0.f, FC_ERR_INVALID_VALUE,
             "fc_varlen_bidir_attention: softmax_scale must be > 0");
  FC_REQUIRE(workspace_bytes >= fc_attention_workspace_size(B, 0, T_k, n_heads, head_dim,
                                                            importance != nullptr),
             FC_ERR_WORKSPACE, "fc_varlen_bidir_attention: workspace too small");
  if (max_seqlen_q == 0) return FC_OK;
  hipStream_t st = (hipStream_t)stream;
  const int log2ps = fc_log2i(page_size);
  if (dtype == FC_DTYPE_BF16) {
    FC_REQUIRE(head_dim == AD, FC_ERR_UNSUPPORTED,
               "fc_varlen_bidir_attention: bf16 needs head_dim 128 (got %d)", head_dim);
    AttnArgs a;
    a.q = (const uint16_t*)q;
    a.kc = (const uint16_t*)k_cache;
    a.vc = (const uint16_t*)v_cache;
    a.block_table = block_table;
    a.cu_q = cu_seqlens_q;
    a.cu_k = cu_seqlens_k;
    a.out = (uint16_t*)out;
    a.imp = importance;
    a.maxp = max_pages_per_seq;
    a.log2ps = log2ps;
    a.B = B;
    a.H = n_heads;
    a.T_k = T_k;
    a.n_rt = (max_seqlen_q + AROWS - 1) / AROWS;
    a.accumulate = accumulate ? 1 : 0;
    a.scale_log2 = softmax_scale * LOG2E;
    if (importance) {
      hipLaunchKernelGGL(attn_bf16_d128<true>, dim3(B * n_heads), dim3(256), 0, st, a);
    } else {
      hipLaunchKernelGGL(attn_bf16_d128<false>, dim3(B * n_heads * a.n_rt), dim3(256), 0, st, a);
    }
    return fc_check_launch("fc_varlen_bidir_attention");
  }
  FC_REQUIRE(head_dim == 64 || head_dim == 128, FC_ERR_UNSUPPORTED,
             "fc_varlen_bidir_attention: f32 needs head_dim 64 or 128 (got %d)", head_dim);
  const size_t shm = (size_t)(2 * F_KT * head_dim + F_ROWS * F_KT) * sizeof(float);
  hipLaunchKernelGGL(attn_f32, dim3(B * n_heads), dim3(F_ROWS), shm, st, (const float*)q,
                     (const float*)k_cache, (const float*)v_cache, block_table, max_pages_per_seq,
                     log2ps, cu_seqlens_q, cu_seqlens_k, n_heads, head_dim, softmax_scale,
                     (float*)out, importance, T_k, accumulate ? 1 : 0);
  return fc_check_launch("fc_varlen_bidir_attention");
}
