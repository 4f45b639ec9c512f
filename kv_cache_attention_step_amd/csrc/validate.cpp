// Checks of the index inputs of a step (query positions, sequence offsets,
// page table) on a host copy, for debugging: fc_validate_step_inputs, and the
// FC_DEBUG checks the step's entry points run before they enqueue anything.
//
// The kernels trust these inputs: a position outside its sequence, two rows of
// one sequence on the same position (their cache writes race) or a page id
// outside the cache would make them read or write outside the caller's
// buffers. Checking them needs their values, so the checks wait for the
// caller's stream (earlier work on it may still be producing them) and copy
// them to the host.
#include <stdlib.h>

#include <algorithm>
#include <vector>

#include "fc_common.hpp"

namespace {

// Copies n int32 values from device memory after the stream's earlier work.
fc_status_t fetch(const int32_t* src, size_t n, hipStream_t st, std::vector<int32_t>& out,
                  const char* what) {
  out.assign(n, 0);
  if (n == 0) return FC_OK;
  hipError_t e = hipMemcpyAsync(out.data(), src, n * sizeof(int32_t), hipMemcpyDeviceToHost, st);
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  if (e != hipSuccess)
    return fc_fail(FC_ERR_HIP, "%s: reading back inputs failed: %s", what, hipGetErrorString(e));
  return FC_OK;
}

fc_status_t check_offsets(const std::vector<int32_t>& cu, int B, int total, const char* name,
                          const char* what) {
  if (cu[0] != 0)
    return fc_fail(FC_ERR_INVALID_VALUE, "%s: %s[0] = %d, must be 0", what, name, cu[0]);
  for (int b = 0; b < B; ++b)
    if (cu[b + 1] < cu[b])
      return fc_fail(FC_ERR_INVALID_VALUE, "%s: %s decreases at sequence %d (%d -> %d)", what,
                     name, b, cu[b], cu[b + 1]);
  if (total >= 0 && cu[B] != total)
    return fc_fail(FC_ERR_INVALID_VALUE, "%s: %s[B] = %d, expected %d", what, name, cu[B], total);
  return FC_OK;
}

// Page-table entries a sequence of length L uses: pages 0 .. ceil(L / ps) - 1.
fc_status_t check_pages(const std::vector<int32_t>& bt, int b, int64_t L, int maxp, int ps,
                        int num_pages, const char* what) {
  const int64_t n = (L + ps - 1) / ps;
  if (n > maxp)
    return fc_fail(FC_ERR_INVALID_VALUE,
                   "%s: sequence %d needs %lld pages of %d, max_pages_per_seq is %d", what, b,
                   (long long)n, ps, maxp);
  for (int64_t j = 0; j < n; ++j) {
    const int32_t page = bt[(size_t)b * maxp + j];
    if (page < 0 || (num_pages > 0 && page >= num_pages))
      return fc_fail(FC_ERR_INVALID_VALUE,
                     "%s: block_table[%d][%lld] = %d is not a page id (num_pages %d)", what, b,
                     (long long)j, page, num_pages);
  }
  return FC_OK;
}

// Rows of sequence b: positions >= 0, < L (when known), distinct (when asked).
fc_status_t check_positions(const std::vector<int32_t>& pos, int b, int q0, int q1, int64_t L,
                            bool distinct, const char* what) {
  for (int t = q0; t < q1; ++t) {
    if (pos[t] < 0 || (L >= 0 && pos[t] >= L))
      return fc_fail(FC_ERR_INVALID_VALUE, "%s: positions[%d] = %d outside sequence %d (length %lld)",
                     what, t, pos[t], b, (long long)L);
  }
  if (distinct && q1 - q0 > 1) {
    std::vector<int32_t> s(pos.begin() + q0, pos.begin() + q1);
    std::sort(s.begin(), s.end());
    for (size_t i = 1; i < s.size(); ++i)
      if (s[i] == s[i - 1])
        return fc_fail(FC_ERR_INVALID_VALUE,
                       "%s: position %d appears twice in sequence %d (its cache writes would race)",
                       what, s[i], b);
  }
  return FC_OK;
}

}  // namespace

bool fc_debug_enabled() {
  const char* v = getenv("FC_DEBUG");
  return v && v[0] && !(v[0] == '0' && v[1] == 0);
}

fc_status_t fc_debug_check_qkv(const int32_t* positions, const int32_t* cu_seqlens_q, int B,
                               int T_q, const int32_t* block_table, int maxp, int page_size,
                               bool write_cache, hipStream_t st) {
  const char* what = "fc_qkv_rope_cache_write (FC_DEBUG)";
  std::vector<int32_t> cu, pos, bt;
  fc_status_t s;
  if ((s = fetch(cu_seqlens_q, (size_t)B + 1, st, cu, what)) != FC_OK) return s;
  if ((s = check_offsets(cu, B, T_q, "cu_seqlens_q", what)) != FC_OK) return s;
  if ((s = fetch(positions, (size_t)T_q, st, pos, what)) != FC_OK) return s;
  if (block_table && (s = fetch(block_table, (size_t)B * maxp, st, bt, what)) != FC_OK) return s;
  for (int b = 0; b < B; ++b) {
    if ((s = check_positions(pos, b, cu[b], cu[b + 1], -1, write_cache, what)) != FC_OK) return s;
    if (!block_table) continue;
    // the page of every row's position must be a page id
    int64_t need = 0;
    for (int t = cu[b]; t < cu[b + 1]; ++t) need = std::max<int64_t>(need, (int64_t)pos[t] + 1);
    if ((s = check_pages(bt, b, need, maxp, page_size, 0, what)) != FC_OK) return s;
  }
  return FC_OK;
}

fc_status_t fc_debug_check_attention(const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                                     int B, int max_seqlen_q, int T_k,
                                     const int32_t* block_table, int maxp, int page_size,
                                     hipStream_t st) {
  const char* what = "fc_varlen_bidir_attention (FC_DEBUG)";
  std::vector<int32_t> cq, ck, bt;
  fc_status_t s;
  if ((s = fetch(cu_seqlens_q, (size_t)B + 1, st, cq, what)) != FC_OK) return s;
  if ((s = fetch(cu_seqlens_k, (size_t)B + 1, st, ck, what)) != FC_OK) return s;
  if ((s = check_offsets(cq, B, -1, "cu_seqlens_q", what)) != FC_OK) return s;
  if ((s = check_offsets(ck, B, T_k, "cu_seqlens_k", what)) != FC_OK) return s;
  if ((s = fetch(block_table, (size_t)B * maxp, st, bt, what)) != FC_OK) return s;
  for (int b = 0; b < B; ++b) {
    if (cq[b + 1] - cq[b] > max_seqlen_q)
      return fc_fail(FC_ERR_INVALID_VALUE, "%s: sequence %d has %d query rows > max_seqlen_q %d",
                     what, b, cq[b + 1] - cq[b], max_seqlen_q);
    if ((s = check_pages(bt, b, ck[b + 1] - ck[b], maxp, page_size, 0, what)) != FC_OK) return s;
  }
  return FC_OK;
}

fc_status_t fc_debug_check_offsets(const int32_t* cu, int B, int total, const char* name,
                                   const char* what, hipStream_t st) {
  std::vector<int32_t> c;
  fc_status_t s;
  if ((s = fetch(cu, (size_t)B + 1, st, c, what)) != FC_OK) return s;
  return check_offsets(c, B, total, name, what);
}

fc_status_t fc_debug_check_views(const int32_t* cu_seqlens_k, const int32_t* verify_start,
                                 int B, const int32_t* block_table, int maxp, int page_size,
                                 int pages_per_view, hipStream_t st) {
  const char* what = "fv_fork_view_pages (FC_DEBUG)";
  std::vector<int32_t> ck, vs, bt;
  fc_status_t s;
  if ((s = fetch(cu_seqlens_k, (size_t)B + 1, st, ck, what)) != FC_OK) return s;
  if ((s = check_offsets(ck, B, -1, "cu_seqlens_k", what)) != FC_OK) return s;
  if ((s = fetch(verify_start, (size_t)B, st, vs, what)) != FC_OK) return s;
  if ((s = fetch(block_table, (size_t)B * maxp, st, bt, what)) != FC_OK) return s;
  for (int b = 0; b < B; ++b) {
    const int L = ck[b + 1] - ck[b];
    if (vs[b] < 0 || vs[b] > L)
      return fc_fail(FC_ERR_INVALID_VALUE, "%s: verify_start[%d] = %d outside [0, %d]", what, b,
                     vs[b], L);
    const int n_pages = (L + page_size - 1) / page_size, first = vs[b] / page_size;
    if (n_pages > maxp)
      return fc_fail(FC_ERR_INVALID_VALUE, "%s: sequence %d needs %d pages > max_pages_per_seq %d",
                     what, b, n_pages, maxp);
    if (n_pages - first > pages_per_view)
      return fc_fail(FC_ERR_INVALID_VALUE,
                     "%s: sequence %d verifies %d pages, more than pages_per_view %d", what, b,
                     n_pages - first, pages_per_view);
    for (int j = 0; j <= first && j < n_pages; ++j)
      if (bt[(size_t)b * maxp + j] < 0)
        return fc_fail(FC_ERR_INVALID_VALUE, "%s: block_table[%d][%d] = %d", what, b, j,
                       bt[(size_t)b * maxp + j]);
  }
  return FC_OK;
}

extern "C" fc_status_t fc_validate_step_inputs(const int32_t* positions,
                                               const int32_t* cu_seqlens_q,
                                               const int32_t* cu_seqlens_k, int32_t B,
                                               int32_t T_q, int32_t T_k,
                                               const int32_t* block_table,
                                               int32_t max_pages_per_seq, int32_t page_size,
                                               int32_t num_pages, fc_stream_t stream) {
  fc_clear_error();
  const char* what = "fc_validate_step_inputs";
  FC_REQUIRE(B >= 1 && T_q >= 0 && T_k >= 0 && max_pages_per_seq >= 1 && num_pages >= 1,
             FC_ERR_INVALID_VALUE, "%s: bad sizes B=%d T_q=%d T_k=%d max_pages_per_seq=%d num_pages=%d",
             what, B, T_q, T_k, max_pages_per_seq, num_pages);
  FC_REQUIRE(fc_is_pow2(page_size) && page_size <= 256, FC_ERR_INVALID_VALUE,
             "%s: page_size=%d must be a power of two <= 256", what, page_size);
  FC_REQUIRE(cu_seqlens_q && cu_seqlens_k && block_table, FC_ERR_INVALID_VALUE,
             "%s: NULL required pointer", what);
  hipStream_t st = (hipStream_t)stream;
  std::vector<int32_t> cq, ck, pos, bt;
  fc_status_t s;
  if ((s = fetch(cu_seqlens_q, (size_t)B + 1, st, cq, what)) != FC_OK) return s;
  if ((s = fetch(cu_seqlens_k, (size_t)B + 1, st, ck, what)) != FC_OK) return s;
  if ((s = check_offsets(cq, B, T_q, "cu_seqlens_q", what)) != FC_OK) return s;
  if ((s = check_offsets(ck, B, T_k, "cu_seqlens_k", what)) != FC_OK) return s;
  if (positions && (s = fetch(positions, (size_t)T_q, st, pos, what)) != FC_OK) return s;
  if ((s = fetch(block_table, (size_t)B * max_pages_per_seq, st, bt, what)) != FC_OK) return s;
  for (int b = 0; b < B; ++b) {
    const int64_t L = ck[b + 1] - ck[b];
    if ((s = check_pages(bt, b, L, max_pages_per_seq, page_size, num_pages, what)) != FC_OK) return s;
    if (positions && (s = check_positions(pos, b, cq[b], cq[b + 1], L, true, what)) != FC_OK) return s;
  }
  return FC_OK;
}
