// Internal declarations shared by the liblsh translation units.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lsh {

// Key tile of the attention kernels (keys per online-softmax step).
constexpr int kBN = 64;
// Head dimension supported by the kernels.
constexpr int kD = 128;
// Query rows per wavefront (one 32x32 MFMA block).
constexpr int kQW = 32;
// Mask block edge of the block-sparse kernel.
constexpr int kMaskBlock = 128;

// Kernel-side description of one attention launch. Strides are in
// elements. LSE of (b, h, s) lives at lse[b * lse_sb + h * lse_sh + s].
struct AttnParams {
  const void* q;
  const void* k;
  const void* v;
  float* o;
  float* lse;
  int64_t q_sb, q_ss, q_sh;
  int64_t k_sb, k_ss, k_sh;
  int64_t v_sb, v_ss, v_sh;
  int64_t o_sb, o_ss, o_sh;
  int64_t lse_sb, lse_sh;
  int32_t B, H, Sq, Skv;
  float scale;        // score multiplier
  float scale_log2;   // scale * log2(e)
  int32_t n_qblk;     // query blocks per (b, h)
  int32_t n_items;    // grid size in work items
  // block-sparse only
  const uint8_t* mask;      // [B, H, n_mqb, n_mkb]
  int32_t n_mqb, n_mkb;
  const int32_t* order;     // work order over items, or nullptr
  const int32_t* counts;    // kept key blocks of each item's mask row
  const unsigned short* kept;   // [n_items][n_mkb]: each row's kept key blocks, ascending
  // nonzero: merge into the (O, LSE) already in o / lse (one ring round
  // folded into a running result) instead of overwriting them
  int32_t accumulate;
  int32_t n_cu;       // compute units of the device (0: assume 256)
  // dense 256-row launches: the last n_tail items of each XCD's range run
  // as two 128-row halves (0: none)
  int32_t n_tail;
};

enum class DType : int { F32 = 0, BF16 = 1 };

// Launchers (return the launch's hipError_t).
hipError_t launch_attn_dense(const AttnParams& p, DType dt, hipStream_t s);
hipError_t launch_attn_sparse(const AttnParams& p, DType dt, hipStream_t s);
hipError_t launch_attn_empty(const AttnParams& p, hipStream_t s);
hipError_t launch_head_permute(const void* src, void* dst, int elem_bytes,
                               int64_t B, int64_t S, int64_t H, int64_t D,
                               int32_t h0, int32_t hc, hipStream_t s);
hipError_t launch_lse_merge(const float* o_parts, const float* lse_parts, int32_t n,
                            int64_t B, int64_t Sq, int64_t H, float* o, float* lse,
                            hipStream_t s);
// Kept-block counts and lists per item, totals per head, the heads' XCD
// placement (heads + 8 entries) and the launch order of the block-sparse
// items (per = query blocks per head; n_items = heads * per).
hipError_t launch_sparse_schedule(const uint8_t* mask, int32_t n_items, int32_t n_mkb, int32_t per,
                                  int32_t* counts, long long* totals, int32_t* order,
                                  unsigned short* kept, int32_t* place, hipStream_t s);

// Query rows per tile of the backward's per-row workspace (and of the
// dK/dV kernel's query loop).
constexpr int kBwdQT = 64;

// Kernel-side description of one attention backward (bf16 Q, K, V, dO;
// float32 O, LSE and gradients). Strides are in elements.
struct BwdParams {
  const void* q;
  const void* k;
  const void* v;
  const void* dout;
  const float* o;
  const float* lse;
  float* dq;
  float* dk;
  float* dv;
  // Per query row, tile by tile: aux[(b*H + h)*n_qt + t][0..63] = LSE *
  // log2(e) of rows 64 t .. 64 t + 63 (+inf past Sq), [64..127] =
  // rowsum(dO * O) of the same rows (0 past Sq).
  float* aux;
  int64_t q_sb, q_ss, q_sh;
  int64_t k_sb, k_ss, k_sh;
  int64_t v_sb, v_ss, v_sh;
  int64_t do_sb, do_ss, do_sh;
  int64_t o_sb, o_ss, o_sh;
  int64_t dq_sb, dq_ss, dq_sh;
  int64_t dk_sb, dk_ss, dk_sh;
  int64_t dv_sb, dv_ss, dv_sh;
  int64_t lse_sb, lse_sh;
  int32_t B, H, Sq, Skv;
  float scale;        // score multiplier
  float scale_log2;   // scale * log2(e)
  int32_t n_qt;       // ceil(Sq / kBwdQT)
  int32_t n_cu;       // compute units of the device (0: assume 256)
};

// Whether the kernel on workgroups of 2R rows (items_big of them) should
// run rather than the one on workgroups of R rows (items_small), judged by
// the rounds each needs over the CUs: a workgroup of the former takes about
// 5/3 as long as one of the latter (twice the rows at about 1.2 times the
// rate), so it wins unless its last round leaves many CUs idle.
inline bool prefer_two_waves(int64_t items_big, int64_t items_small, int n_cu) {
  const int64_t cus = n_cu > 0 ? n_cu : 256;
  const int64_t r_big = (items_big + cus - 1) / cus;
  const int64_t r_small = (items_small + cus - 1) / cus;
  return 5 * r_big <= 3 * r_small;
}

// Workgroups go to the 8 XCDs in turn, and the dense kernels give XCD x the
// contiguous items x * per .. x * per + per - 1 (per = items / 8). With one
// 256-row workgroup per CU, an XCD's last round holds per % (CUs per XCD)
// of them and leaves the other CUs idle. When that remainder is at most
// half an XCD's CUs, running those items as twice as many 128-row halves
// (about 3/5 of the time each) ends the round sooner. Returns the number of
// items per XCD to split, or 0 (also when the items or the CUs do not split
// evenly over the XCDs).
inline int32_t tail_halves(int64_t items_big, int n_cu) {
  constexpr int64_t kX = 8;
  const int64_t cus = n_cu > 0 ? n_cu : 256;
  if (cus % kX != 0 || items_big % kX != 0) return 0;
  const int64_t per = items_big / kX, cu_x = cus / kX;
  const int64_t r = per % cu_x;
  return (r > 0 && 2 * r <= cu_x && per > cu_x) ? (int32_t)r : 0;
}

// Enqueues the three backward kernels (row statistics, dK/dV, dQ).
hipError_t launch_attn_bwd(const BwdParams& p, hipStream_t s);
// Enqueues the dQ kernel alone (the last of the three).
hipError_t launch_attn_bwd_dq(const BwdParams& p, hipStream_t s);

}  // namespace lsh
