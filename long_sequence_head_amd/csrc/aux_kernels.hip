// Memory-bound companions of the attention kernels: the head-major copy
// that stands in for the Ulysses all-to-all, the log-sum-exp merge of
// per-KV-block partial results, and the work order of the block-sparse
// kernel.
#include "attn_common.hpp"

namespace lsh {
namespace {

// ------------------------------------------------------------ head permute
//
// dst[b, h - h0, s, :] = src[b, s, h, :] for h in [h0, h0 + hc): the local
// re-layout an all-to-all performs when sequence sharding turns into head
// sharding ("HCMS: Head-Chunked Multi-Stream Pipeline ...", Abstract). Rows
// are copied as 16-byte chunks. blockIdx.y = b * hc + (h - h0) selects the
// destination row group, whose S rows are contiguous; each thread moves
// kUnroll chunks, all loads issued before the stores.
constexpr int kPermThreads = 256;
constexpr int kPermUnroll = 4;

__global__ __launch_bounds__(kPermThreads) void head_permute_kernel(
    const u32x4* __restrict__ src, u32x4* __restrict__ dst, int S, int H, int cpr, int cpr_shift,
    int h0, int hc) {
  const int bh = blockIdx.y;
  const int b = bh / hc, hr = bh - b * hc;
  const unsigned n_chunks = (unsigned)S * (unsigned)cpr;  // chunks in this row group (< 2^31)
  const u32x4* srow = src + ((int64_t)b * S * H + h0 + hr) * cpr;  // (s = 0, c = 0)
  u32x4* drow = dst + (int64_t)bh * n_chunks;
  const int64_t src_row_stride = (int64_t)H * cpr;
  const unsigned base = blockIdx.x * (unsigned)(kPermThreads * kPermUnroll) + threadIdx.x;
  u32x4 v[kPermUnroll];
#pragma unroll
  for (int u = 0; u < kPermUnroll; ++u) {
    const unsigned i = base + u * kPermThreads;
    if (i < n_chunks) {
      const unsigned s = cpr_shift >= 0 ? (i >> cpr_shift) : i / (unsigned)cpr;
      const unsigned c = i - s * (unsigned)cpr;
      v[u] = __builtin_nontemporal_load(srow + s * src_row_stride + c);
    }
  }
#pragma unroll
  for (int u = 0; u < kPermUnroll; ++u) {
    const unsigned i = base + u * kPermThreads;
    if (i < n_chunks) __builtin_nontemporal_store(v[u], drow + i);
  }
}

// ---------------------------------------------------------------- LSE merge
//
// Partial results over disjoint key sets, each normalised over its own
// keys with its log-sum-exp, combine into the result over the union:
// M = max_k LSE_k, w_k = exp(LSE_k - M), Z = sum_k w_k, LSE = M + log Z,
// O = sum_k (w_k / Z) O_k. Ring Attention accumulates per-block results
// this way ("CHARM+: How Cross-Hardware Attention Breaks Through
// Distributed Communication Bottlenecks", section on the communication
// bottleneck). One (b, s, h) row of 128 floats per 32 lanes, float4 each;
// consecutive rows are contiguous in O.
//
// HBM-bound: a lane issues the loads of a whole group of up to kMergeGroup
// partials (their LSE and its 16 bytes of each O) before it uses any of
// them, so one memory round trip serves the group. Groups after the first
// fold in with the running max: when a group raises M, what was summed so
// far is scaled by exp(M_old - M_new). The sums run over k = 0, 1, ... in
// order.
constexpr int kMergeThreads = 128;
constexpr int kMergeGroup = 8;

__global__ __launch_bounds__(kMergeThreads) void lse_merge_kernel(
    const float* __restrict__ o_parts, const float* __restrict__ lse_parts, int n, int B, int Sq,
    int H, float* __restrict__ o, float* __restrict__ lse) {
  const unsigned rows = (unsigned)B * (unsigned)Sq * (unsigned)H;  // < 2^31
  // XCD-aware block order: the blocks one XCD runs take consecutive rows,
  // so that XCD's L2 serves each 64-byte line of the LSE arrays (16
  // consecutive s of one h) to all the rows that use it
  const unsigned row = (unsigned)xcd_remap((int)blockIdx.x, (int)gridDim.x) * (unsigned)(kMergeThreads / 32) +
                       (threadIdx.x >> 5);
  const int l = threadIdx.x & 31;
  if (row >= rows) return;
  const unsigned bs = row / (unsigned)H;
  const int h = (int)(row - bs * (unsigned)H);
  const unsigned b_ = bs / (unsigned)Sq;
  const int s = (int)(bs - b_ * (unsigned)Sq);
  const int b = (int)b_;
  const int64_t lse_off = ((int64_t)b * H + h) * Sq + s;  // within one part
  const int64_t lse_step = (int64_t)B * H * Sq;
  const int64_t o_step = (int64_t)rows * kD;
  const f32x4* op = reinterpret_cast<const f32x4*>(o_parts + (int64_t)row * kD) + l;

  float M = kNegInf, Z = 0.0f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int k0 = 0; k0 < n; k0 += kMergeGroup) {
    // Every slot of the group loads (slots past the last partial reload
    // that one and get weight 0 through LSE = -inf): branch-free, so the
    // loads are all in flight at once.
    f32x4 ok[kMergeGroup];
    float w[kMergeGroup];
#pragma unroll
    for (int j = 0; j < kMergeGroup; ++j) {
      const int kk = k0 + j < n ? k0 + j : n - 1;
      w[j] = lse_parts[kk * lse_step + lse_off];
      ok[j] = __builtin_nontemporal_load(op + kk * (o_step / 4));
    }
#pragma unroll
    for (int j = 0; j < kMergeGroup; ++j) w[j] = k0 + j < n ? w[j] : kNegInf;
    float mg = kNegInf;
#pragma unroll
    for (int j = 0; j < kMergeGroup; ++j) mg = fmaxf(mg, w[j]);
    // Branch-free, so that nothing holds the loads back: while every part
    // so far is empty (M = -inf) the exponents use 0 and every weight is 0;
    // r is exactly 1 when the group does not raise M.
    const float m_new = fmaxf(M, mg);
    const float m_use = m_new == kNegInf ? 0.0f : m_new;
    const float r = __expf(M - m_use);
    Z *= r;
    acc *= r;
    M = m_new;
#pragma unroll
    for (int j = 0; j < kMergeGroup; ++j) {
      const float wj = __expf(w[j] - m_use);   // 0 for an empty part or a padding slot
      acc += wj * ok[j];
      Z += wj;
    }
  }
  float out_lse = kNegInf;
  if (M != kNegInf) {
    acc *= 1.0f / Z;
    out_lse = M + __logf(Z);
  }
  __builtin_nontemporal_store(acc, reinterpret_cast<f32x4*>(o + (int64_t)row * kD) + l);
  if (l == 0) lse[lse_off] = out_lse;
}

// ------------------------------------------------------ block-sparse order
//
// Work items are the (b, h, query-block) rows of the block mask. Heads
// differ in density and dense blocks sit irregularly ("db-SP: Accelerating
// Sparse Attention for Visual Generative Models with Dual-Balanced Sequence
// Parallelism", Abstract), so items are launched heaviest first (longest
// processing time first): the hardware dispatcher then fills CUs greedily
// and the light items pack the tail.

// counts[item] = number of kept key blocks in the item's mask row, and
// kept[item][0 .. counts[item]) = those blocks' indices, ascending (one
// wavefront per row: a ballot per 64 blocks, each kept block's slot is the
// number of kept blocks before it).
__global__ __launch_bounds__(256) void sparse_count_kernel(const uint8_t* __restrict__ mask,
                                                           int n_items, int n_mkb,
                                                           int* __restrict__ counts,
                                                           unsigned short* __restrict__ kept) {
  const int item = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (item >= n_items) return;
  const uint8_t* row = mask + (int64_t)item * n_mkb;
  unsigned short* krow = kept + (int64_t)item * n_mkb;
  int cnt = 0;
  for (int base = 0; base < n_mkb; base += 64) {
    const int j = base + lane;
    const bool flag = j < n_mkb && row[j] != 0;
    const unsigned long long bal = __ballot(flag);
    if (flag) krow[cnt + __builtin_popcountll(bal & ((1ull << lane) - 1ull))] = (unsigned short)j;
    cnt += __builtin_popcountll(bal);
  }
  if (lane == 0) counts[item] = cnt;
}

// Launch order of the block-sparse work items. Item i = g * per + r is
// query block r of head g = b * H + h. Launch slots go to the 8 XCDs in
// turn (slot s runs on XCD s mod 8), so the order decides what each XCD's
// L2 sees. Heads are dealt to the XCDs whole, by kept-block total: in
// descending total (ties: lower head index first), each head goes to the
// XCD with the smallest total so far among those holding fewer than
// ceil(G / 8) heads (ties: lowest XCD), so every head's K/V is streamed
// through one XCD's L2 and the XCDs carry about equal work. Each XCD's list
// is its heads in the order dealt, each head's query blocks in descending
// kept count (ties: lower index first): the XCD works through one head's
// rows at a time, heaviest first. Position j of XCD x's list (lists of
// L_x items) takes slot sum_x' min(L_x', j) + #{x' < x : L_x' > j}, i.e.
// the lists interleave slot by slot (slot 8 j + x while all eight run).
constexpr int kXcds = 8;

// Kept-block total of each head: one wavefront per head (exact integer sum).
__global__ __launch_bounds__(256) void sparse_total_kernel(const int* __restrict__ counts,
                                                           int n_groups, int per,
                                                           long long* __restrict__ totals) {
  const int g = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (g >= n_groups) return;
  const int* c = counts + (int64_t)g * per;
  long long t = 0;
  for (int j = lane; j < per; j += 64) t += c[j];
  for (int off = 32; off >= 1; off >>= 1) t += __shfl_xor(t, off);
  if (lane == 0) totals[g] = t;
}

// Deals the heads to the XCDs (one workgroup): place[g] = x + 8 * k for
// the k-th head dealt to XCD x, place[G + x] = heads of XCD x. The heads'
// descending-total order goes through by_rank (G entries of scratch), with
//   rank(g) = #{k : T_k > T_g} + #{k < g : T_k = T_g}.
__global__ __launch_bounds__(256) void sparse_place_kernel(const long long* __restrict__ totals,
                                                           int n_groups, int* __restrict__ by_rank,
                                                           int* __restrict__ place) {
  for (int g = threadIdx.x; g < n_groups; g += 256) {
    const long long t_g = totals[g];
    int rank = 0;
    for (int k = 0; k < n_groups; ++k) {
      const long long t_k = totals[k];
      rank += (t_k > t_g) | ((t_k == t_g) & (k < g));
    }
    by_rank[rank] = g;
  }
  __syncthreads();
  if (threadIdx.x != 0) return;
  const int cap = (n_groups + kXcds - 1) / kXcds;
  long long load[kXcds];
  int cnt[kXcds];
  for (int x = 0; x < kXcds; ++x) {
    load[x] = 0;
    cnt[x] = 0;
  }
  for (int r = 0; r < n_groups; ++r) {
    const int g = by_rank[r];
    int best = -1;
    for (int x = 0; x < kXcds; ++x)
      if (cnt[x] < cap && (best < 0 || load[x] < load[best])) best = x;
    place[g] = best + kXcds * cnt[best];
    ++cnt[best];
    load[best] += totals[g];
  }
  for (int x = 0; x < kXcds; ++x) place[n_groups + x] = cnt[x];
}

// order[slot(g, r)] = g * per + r with j = per * k(g) + rank_g(r), where
//   rank_g(r) = #{j : c_j > c_r} + #{j < r : c_j = c_r} over the head's
//               query blocks (c = counts),
// and the slot of position j of XCD x(g) as above. A workgroup ranks 256
// query blocks of one head, reading the head's counts from LDS in chunks
// (every lane reads the same entry: a broadcast).
constexpr int kOrderThreads = 256;
constexpr int kOrderChunk = 4096;

__global__ __launch_bounds__(kOrderThreads) void sparse_order_kernel(
    const int* __restrict__ counts, const int* __restrict__ place, int n_groups, int per,
    int* __restrict__ order) {
  __shared__ int cbuf[kOrderChunk];
  const int blocks_per_group = (per + kOrderThreads - 1) / kOrderThreads;
  const int g = blockIdx.x / blocks_per_group;
  const int r = (blockIdx.x % blocks_per_group) * kOrderThreads + threadIdx.x;
  const int* c = counts + (int64_t)g * per;
  const int c_r = r < per ? c[r] : 0;
  int lr = 0;
  for (int base = 0; base < per; base += kOrderChunk) {
    const int m = per - base < kOrderChunk ? per - base : kOrderChunk;
    __syncthreads();
    for (int j = threadIdx.x; j < m; j += kOrderThreads) cbuf[j] = c[base + j];
    __syncthreads();
    for (int j = 0; j < m; ++j) {
      const int c_j = cbuf[j];
      lr += (c_j > c_r) | ((c_j == c_r) & (base + j < r));
    }
  }
  if (r >= per) return;
  const int pl = place[g];
  const int x = pl % kXcds;
  const long long j = (long long)per * (pl / kXcds) + lr;
  long long slot = 0;
  for (int x2 = 0; x2 < kXcds; ++x2) {
    const long long len = (long long)per * place[n_groups + x2];
    slot += len < j ? len : j;
    if (x2 < x && len > j) ++slot;
  }
  order[slot] = g * per + r;
}

}  // namespace

hipError_t launch_head_permute(const void* src, void* dst, int elem_bytes, int64_t B, int64_t S,
                               int64_t H, int64_t D, int32_t h0, int32_t hc, hipStream_t s) {
  const int cpr = (int)(D * elem_bytes / 16);
  const int cpr_shift = (cpr & (cpr - 1)) == 0 ? __builtin_ctz((unsigned)cpr) : -1;
  const int64_t n_chunks = S * cpr;
  const int64_t per_block = kPermThreads * kPermUnroll;
  dim3 grid((unsigned)((n_chunks + per_block - 1) / per_block), (unsigned)(B * hc));
  hipLaunchKernelGGL(head_permute_kernel, grid, dim3(kPermThreads), 0, s,
                     static_cast<const u32x4*>(src), static_cast<u32x4*>(dst), (int)S, (int)H, cpr,
                     cpr_shift, h0, hc);
  return hipGetLastError();
}

hipError_t launch_lse_merge(const float* o_parts, const float* lse_parts, int32_t n, int64_t B,
                            int64_t Sq, int64_t H, float* o, float* lse, hipStream_t s) {
  const int64_t rows = B * Sq * H;
  const int64_t rpb = kMergeThreads / 32;
  hipLaunchKernelGGL(lse_merge_kernel, dim3((unsigned)((rows + rpb - 1) / rpb)),
                     dim3(kMergeThreads), 0, s, o_parts, lse_parts, n, (int)B, (int)Sq, (int)H, o,
                     lse);
  return hipGetLastError();
}

hipError_t launch_sparse_schedule(const uint8_t* mask, int32_t n_items, int32_t n_mkb, int32_t per,
                                  int32_t* counts, long long* totals, int32_t* order,
                                  unsigned short* kept, int32_t* place, hipStream_t s) {
  hipLaunchKernelGGL(sparse_count_kernel, dim3((n_items + 3) / 4), dim3(256), 0, s, mask, n_items,
                     n_mkb, counts, kept);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int n_groups = n_items / per;
  hipLaunchKernelGGL(sparse_total_kernel, dim3((n_groups + 3) / 4), dim3(256), 0, s, counts,
                     n_groups, per, totals);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  // the order array is scratch for the heads' rank order until the order
  // kernel overwrites it
  hipLaunchKernelGGL(sparse_place_kernel, dim3(1), dim3(256), 0, s, totals, n_groups, order, place);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int blocks_per_group = (per + kOrderThreads - 1) / kOrderThreads;
  hipLaunchKernelGGL(sparse_order_kernel, dim3((unsigned)((int64_t)n_groups * blocks_per_group)),
                     dim3(kOrderThreads), 0, s, counts, place, n_groups, per, order);
  return hipGetLastError();
}

}  // namespace lsh
