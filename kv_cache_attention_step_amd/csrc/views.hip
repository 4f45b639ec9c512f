// Flash-Verify's two views with view-private K/V, and the commit of the
// accepted tokens' K/V into the shared cache.
//
// Drafts and [MASK] tokens are checked through two views of the same
// positions, and predictions that meet the confidence threshold are accepted
// together (infernews post "Flash-dLLM 讓擴散式語言模型解碼更快、更省記憶體",
// paragraph 3; the scheme is a KV-cache-driven draft-and-verify: fugumt
// abstract page). Each view projects its own rows, so each view sees its own
// fresh K/V at the verified positions and the shared cache everywhere else;
// the two views cannot share one cache write.
//
// Design: no new attention kernel. Each (sequence b, view v) becomes a
// virtual sequence 2b + v whose block-table row shares b's pages before the
// verified block and points at private pages (reserved at the end of the
// cache arrays, pages_per_view of them per virtual sequence) from the page
// holding the first verified position on. fv_fork_view_pages builds those rows
// and copies the shared part of that first page into the private page; the
// fused projection then writes each view's fresh K/V into its private pages
// and the one-pass attention runs over the 2B virtual sequences.
// fv_commit_accepted copies, for every accepted position, the draft view's
// K/V rows into the sequence's shared slot.
#include "fc_common.hpp"

namespace {

// One workgroup per (virtual sequence s = 2b + v, head h): head 0's writes the
// view's table row; each copies its head's part of the first private page.
__global__ __launch_bounds__(256) void fork_kernel(
    const int32_t* __restrict__ block_table, int maxp, int log2ps,
    const int32_t* __restrict__ cu_k, const int32_t* __restrict__ verify_start,
    int view_page_base, int pages_per_view, int32_t* __restrict__ view_table,
    uint16_t* __restrict__ kc, uint16_t* __restrict__ vc, int H) {
  const int s = blockIdx.x, b = s >> 1, h = blockIdx.y;
  const int ps = 1 << log2ps;
  const int L = cu_k[b + 1] - cu_k[b];
  const int vs = verify_start[b];
  const int first_pg = vs >> log2ps;
  const int n_pages = (L + ps - 1) >> log2ps;
  const int priv0 = view_page_base + s * pages_per_view;
  const int32_t* src_row = block_table + (size_t)b * maxp;
  if (h == 0) {
    int32_t* dst_row = view_table + (size_t)s * maxp;
    for (int j = threadIdx.x; j < maxp; j += blockDim.x)
      dst_row[j] = j < first_pg ? src_row[j] : (j < n_pages ? priv0 + (j - first_pg) : -1);
  }
  // the shared positions of the first private page: first_pg * ps .. vs - 1;
  // in the [page, head, offset, dim] layout one page is H * ps rows of D
  const int keep = vs - first_pg * ps;
  if (keep <= 0 || first_pg >= n_pages) return;
  const int src_page = src_row[first_pg];
  const size_t page_elems = (size_t)H * ps * 128;
  // rows (h, off) with off < keep; 16-byte chunks, 16 per 128-wide row
  for (int c = threadIdx.x; c < keep * 16; c += blockDim.x) {
    const int ch = c & 15, off = c >> 4;
    const size_t e = ((size_t)h * ps + off) * 128 + ch * 8;
    *(u32x4_t*)(kc + (size_t)priv0 * page_elems + e) = *(const u32x4_t*)(kc + (size_t)src_page * page_elems + e);
    *(u32x4_t*)(vc + (size_t)priv0 * page_elems + e) = *(const u32x4_t*)(vc + (size_t)src_page * page_elems + e);
  }
}

// One workgroup per verified position p (global index over cu_positions).
__global__ __launch_bounds__(256) void commit_kernel(
    const int32_t* __restrict__ block_table, const int32_t* __restrict__ view_table, int maxp,
    int log2ps, const int32_t* __restrict__ cu_p, int B, const int32_t* __restrict__ verify_start,
    const uint8_t* __restrict__ accept_pos, int H, uint16_t* __restrict__ kc,
    uint16_t* __restrict__ vc) {
  const int p = blockIdx.x;
  if (!accept_pos[p]) return;
  int lo = 0, hi = B;  // cu_p[lo] <= p < cu_p[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (cu_p[mid] <= p) lo = mid; else hi = mid;
  }
  const int b = lo;
  const int pos = verify_start[b] + (p - cu_p[b]);
  const int ps = 1 << log2ps, pg = pos >> log2ps, off = pos & (ps - 1);
  const int dst_page = block_table[(size_t)b * maxp + pg];
  const int src_page = view_table[(size_t)(2 * b) * maxp + pg];   // the draft view's page
  const size_t page_elems = (size_t)H * ps * 128;
  // H rows of 128 values, 16 chunks of 8 each
  for (int c = threadIdx.x; c < H * 16; c += blockDim.x) {
    const int h = c >> 4, ch = c & 15;
    const size_t e = ((size_t)h * ps + off) * 128 + ch * 8;
    *(u32x4_t*)(kc + (size_t)dst_page * page_elems + e) = *(const u32x4_t*)(kc + (size_t)src_page * page_elems + e);
    *(u32x4_t*)(vc + (size_t)dst_page * page_elems + e) = *(const u32x4_t*)(vc + (size_t)src_page * page_elems + e);
  }
}

}  // namespace

extern "C" fc_status_t fv_fork_view_pages(void* k_cache, void* v_cache, const int32_t* block_table,
                                          int32_t max_pages_per_seq, int32_t page_size,
                                          const int32_t* cu_seqlens_k,
                                          const int32_t* verify_start, int32_t B,
                                          int32_t n_heads, int32_t head_dim,
                                          int32_t view_page_base, int32_t pages_per_view,
                                          int32_t* view_block_table, fc_stream_t stream) {
  fc_clear_error();
  FC_REQUIRE(B >= 1 && n_heads >= 1 && n_heads <= 65535 && max_pages_per_seq >= 1 &&
                 view_page_base >= 0 && pages_per_view >= 1, FC_ERR_INVALID_VALUE,
             "fv_fork_view_pages: bad sizes B=%d n_heads=%d max_pages_per_seq=%d "
             "view_page_base=%d pages_per_view=%d", B, n_heads, max_pages_per_seq,
             view_page_base, pages_per_view);
  FC_REQUIRE(head_dim == 128, FC_ERR_UNSUPPORTED, "fv_fork_view_pages: head_dim must be 128");
  FC_REQUIRE(fc_is_pow2(page_size) && page_size <= 256, FC_ERR_INVALID_VALUE,
             "fv_fork_view_pages: page_size=%d must be a power of two <= 256", page_size);
  FC_REQUIRE(k_cache && v_cache && block_table && cu_seqlens_k && verify_start && view_block_table,
             FC_ERR_INVALID_VALUE, "fv_fork_view_pages: NULL required pointer");
  FC_REQUIRE(((uintptr_t)k_cache | (uintptr_t)v_cache) % 16 == 0, FC_ERR_INVALID_VALUE,
             "fv_fork_view_pages: caches must be 16-byte aligned");
  FC_REQUIRE((int64_t)view_page_base + 2LL * B * pages_per_view < (1LL << 31), FC_ERR_INVALID_VALUE,
             "fv_fork_view_pages: private page ids overflow int32");
  if (fc_debug_enabled()) {
    const fc_status_t s = fc_debug_check_views(cu_seqlens_k, verify_start, B, block_table,
                                               max_pages_per_seq, page_size, pages_per_view,
                                               (hipStream_t)stream);
    if (s != FC_OK) return s;
  }
  hipLaunchKernelGGL(fork_kernel, dim3(2 * B, n_heads), dim3(256), 0, (hipStream_t)stream,
                     block_table, max_pages_per_seq, fc_log2i(page_size), cu_seqlens_k,
                     verify_start, view_page_base, pages_per_view, view_block_table,
                     (uint16_t*)k_cache, (uint16_t*)v_cache, n_heads);
  return fc_check_launch("fv_fork_view_pages");
}

extern "C" fc_status_t fv_commit_accepted(void* k_cache, void* v_cache, const int32_t* block_table,
                                          const int32_t* view_block_table,
                                          int32_t max_pages_per_seq, int32_t page_size,
                                          const int32_t* cu_positions, const int32_t* verify_start,
                                          int32_t B, int32_t n_positions,
                                          const uint8_t* accept_pos, int32_t n_heads,
                                          int32_t head_dim, fc_stream_t stream) {
  fc_clear_error();
  FC_REQUIRE(B >= 1 && n_heads >= 1 && n_positions >= 0 && max_pages_per_seq >= 1,
             FC_ERR_INVALID_VALUE, "fv_commit_accepted: bad sizes B=%d n_heads=%d n_positions=%d",
             B, n_heads, n_positions);
  FC_REQUIRE(head_dim == 128, FC_ERR_UNSUPPORTED, "fv_commit_accepted: head_dim must be 128");
  FC_REQUIRE(fc_is_pow2(page_size) && page_size <= 256, FC_ERR_INVALID_VALUE,
             "fv_commit_accepted: page_size=%d must be a power of two <= 256", page_size);
  if (n_positions == 0) return FC_OK;
  FC_REQUIRE(k_cache && v_cache && block_table && view_block_table && cu_positions &&
                 verify_start && accept_pos, FC_ERR_INVALID_VALUE,
             "fv_commit_accepted: NULL required pointer");
  FC_REQUIRE(((uintptr_t)k_cache | (uintptr_t)v_cache) % 16 == 0, FC_ERR_INVALID_VALUE,
             "fv_commit_accepted: caches must be 16-byte aligned");
  if (fc_debug_enabled()) {
    const fc_status_t s = fc_debug_check_offsets(cu_positions, B, n_positions, "cu_positions",
                                                 "fv_commit_accepted (FC_DEBUG)", (hipStream_t)stream);
    if (s != FC_OK) return s;
  }
  hipLaunchKernelGGL(commit_kernel, dim3(n_positions), dim3(256), 0, (hipStream_t)stream,
                     block_table, view_block_table, max_pages_per_seq, fc_log2i(page_size),
                     cu_positions, B, verify_start, accept_pos, n_heads, (uint16_t*)k_cache,
                     (uint16_t*)v_cache);
  return fc_check_launch("fv_commit_accepted");
}
