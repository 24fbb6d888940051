// Blockwise online-softmax attention forward for gfx950 (MI355X).
//
// What is computed: for each (b, h) and query row i,
//   LSE_i = log(sum_j exp(scale * <q_i, k_j>)),
//   O_i   = sum_j exp(scale * <q_i, k_j> - LSE_i) * v_j,
// the per-head scaled dot-product attention of "LLM Lab Notes 05: Attention
// Tensor Parallelism - Splitting QKV by Head, Megatron Style" (sections 2
// and 3), over all keys (dense) or over the kept 128x128 blocks of a block
// mask (block-wise sparse attention, "db-SP: Accelerating Sparse Attention
// for Visual Generative Models with Dual-Balanced Sequence Parallelism",
// Abstract).
//
// Design, common to the bf16 kernels (a wavefront owns 32 query rows; the
// wavefronts of a workgroup share each key tile through LDS):
//  * Q of the wavefront's 32 rows stays in registers for the whole key loop.
//  * Key tiles of 64 keys go straight from HBM into LDS slots with
//    buffer_load ... lds. K rows are XOR-swizzled by 16-byte chunk so the
//    QK^T operand reads are bank-conflict free; V rows use a different
//    swizzle matched to the transposing reads below.
//  * S^T = K Q^T on v_mfma_f32_32x32x16_bf16: the accumulator puts one
//    query per lane (lane l and l+32 share query l%32 and split the keys),
//    so the row max and row sum need one cross-half swap only
//    (v_permlane32_swap), and the exponentiated scores are already laid
//    out as the B operand of the next product.
//  * O^T += V^T P^T on the same MFMA. V^T comes straight from the
//    row-major V tile with ds_read_b64_tr_b16, which returns, per lane, 4
//    keys of one head_dim column.
//  * Online softmax in the log2 domain with a lazy rescale: the running
//    max only moves when a tile's max exceeds it by more than 2^8 in
//    probability, so P stays <= 256 and the O rescale is skipped on almost
//    every tile. Each query's arithmetic depends only on its own scores,
//    in an order fixed per query, so results do not depend on the kernel
//    chosen, the workgroup size, the grid order, the number of heads or the
//    strides.
// Two schedules implement it: a ping-pong kernel (two wavefronts per SIMD
// alternating matrix and softmax phases) for large grids, and a
// one-wavefront-per-SIMD software-pipelined kernel for small grids and the
// block-sparse case. fp32 inputs use v_mfma_f32_32x32x2_f32 with the same
// structure and P kept in fp32.
#include "lsh_internal.hpp"

#include <cstring>
#include <type_traits>

namespace lsh {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

#define LDS_AS __attribute__((address_space(3)))

constexpr float kNegInf = -__builtin_inff();
// Lazy-rescale threshold in log2 units: the running max is replaced only
// when a new score exceeds it by more than this.
constexpr float kRescaleLog2 = 8.0f;

// 16-byte chunk swizzles inside a 256-byte (128 x bf16) LDS row.
__device__ __forceinline__ int swz_k(int row, int c) { return c ^ (row & 15); }
__device__ __forceinline__ int swz_v(int row, int c) {
  return c ^ (((row & 3) << 2) | ((row >> 2) & 3));
}

// Workgroups are handed to the 8 XCDs round-robin; remap so that each XCD
// walks a contiguous range of (b, h, query-block) items and the K/V stream
// of a head is shared inside one XCD's L2.
__device__ __forceinline__ int xcd_remap(int bid, int n) {
  constexpr int X = 8;
  const int per = n / X, rem = n % X;
  const int x = bid % X, k = bid / X;
  return x < rem ? x * (per + 1) + k : rem * (per + 1) + (x - rem) * per + k;
}

// Value of lane l^32 (the other half of the wavefront) for both halves:
// r[0] + r[1] / max(r[0], r[1]) combine the two halves.
__device__ __forceinline__ float pair_max(float x) {
  unsigned u = __builtin_bit_cast(unsigned, x);
  auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return fmaxf(__builtin_bit_cast(float, (unsigned)r[0]), __builtin_bit_cast(float, (unsigned)r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  unsigned u = __builtin_bit_cast(unsigned, x);
  auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __builtin_bit_cast(float, (unsigned)r[0]) + __builtin_bit_cast(float, (unsigned)r[1]);
}

__device__ __forceinline__ bool wave_any(bool p) { return __ballot(p) != 0; }

// Item -> (b, h, query block) and the per-item key-tile list.
struct Item {
  int b, h, qblk;
};

__device__ __forceinline__ Item decode_item(int item, int n_qblk, int H) {
  Item it;
  it.qblk = item % n_qblk;
  const int bh = item / n_qblk;
  it.h = bh % H;
  it.b = bh / H;
  return it;
}

// Builds, in LDS, the ascending list of kept key blocks of one mask row.
// Returns the number of kept blocks (same value in every thread).
template <int NT>
__device__ int build_kept_list(const uint8_t* mrow, int n_mkb, unsigned short* kept,
                               int* wave_cnt) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  constexpr int W = NT / 64;
  int total = 0;
  for (int base = 0; base < n_mkb; base += NT) {
    const int j = base + tid;
    const bool flag = j < n_mkb && mrow[j] != 0;
    const unsigned long long bal = __ballot(flag);
    const int below = __builtin_popcountll(bal & ((1ull << lane) - 1ull));
    if (lane == 0) wave_cnt[wave] = __builtin_popcountll(bal);
    __syncthreads();
    int before = 0, sum = 0;
#pragma unroll
    for (int w = 0; w < W; ++w) {
      const int c = wave_cnt[w];
      before += (w < wave) ? c : 0;
      sum += c;
    }
    if (flag) kept[total + before + below] = (unsigned short)j;
    total += sum;
    __syncthreads();
  }
  return total;
}

// Start key of tile t: dense tiles are consecutive; sparse tiles are the two
// 64-key halves of each kept 128-key block.
template <bool SPARSE>
__device__ __forceinline__ int tile_key0(int t, const unsigned short* kept) {
  if constexpr (SPARSE) {
    return (int)kept[t >> 1] * kMaskBlock + (t & 1) * kBN;
  } else {
    return t * kBN;
  }
}

// ------------------------------------------- bf16 dense, ping-pong schedule
//
// The 8 wavefronts of a workgroup form two groups of four, one wavefront of
// each group per SIMD. Every wavefront alternates two phases separated by
// workgroup barriers:
//   Q-phase(t): S(t) = K(t) Q^T                       (16 MFMA, no VALU work)
//   P-phase(t): row max, lazy rescale and exp2 of S(t) -> P(t), interleaved
//               with O^T += V(t-1)^T P(t-1)^T          (16 MFMA, ~130 VALU)
// and group B runs one phase behind group A, so on each SIMD one wavefront
// feeds the matrix core with QK^T while the other one's softmax keeps the
// VALU busy next to its PV products.
//
// K/V tiles stream through a 3-slot LDS ring per tensor, filled with
// buffer_load_dwordx4 ... lds (each lane's 16 bytes land at slot base + 16 *
// lane; loads past the head's last key return zeros: the zero fill of a
// ragged last tile). Intervals between barriers are numbered k = 0, 1, ...;
// K(t) is issued in interval 2t-4 and V(t) in interval 2t-1, so every load
// has two intervals to land; a wavefront waits only for loads issued two
// or more intervals back (s_waitcnt vmcnt) before the barrier, and no fence
// drains the prefetch. A slot is refilled only after the barrier that
// follows its last reader.

constexpr int kStages = 3;
constexpr int kTileBytes = kBN * kD * 2;   // one 64 x 128 bf16 tile

// LDS byte addresses of one tile's K fragments (by d-step) and V^T fragment
// reads (by half and d block).
struct KAddr { uint32_t a[8]; };
struct VAddr { uint32_t a[2][4]; };

// s_waitcnt with vmcnt = N (6 bits: [3:0] and [15:14]); expcnt and lgkmcnt
// left at their maximum.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt out of range");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}

__device__ __forceinline__ void barrier_no_fence() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

template <int WAVES>
__global__ __launch_bounds__(WAVES * 64) void attn_fwd_bf16_pp_kernel(AttnParams p) {
  static_assert(WAVES == 8, "two groups of one wavefront per SIMD");
  constexpr int BM = WAVES * kQW;
  constexpr int LPW = (kTileBytes / 1024) / (WAVES / 2);   // 1-KiB loads per wavefront per tile
  static_assert(LPW >= 1 && LPW * (WAVES / 2) * 1024 == kTileBytes, "tile/threads mismatch");

  __shared__ __attribute__((aligned(1024))) unsigned char lds_k[kStages][kTileBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char lds_v[kStages][kTileBytes];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hh = lane >> 5;
  const bool grp_b = wave >= WAVES / 2;

  const Item it = decode_item(xcd_remap(blockIdx.x, gridDim.x), p.n_qblk, p.H);
  const int qi = it.qblk * BM + wave * kQW + l32;
  const bool q_ok = qi < p.Sq;
  const __bf16* qp = static_cast<const __bf16*>(p.q) + it.b * p.q_sb + it.h * p.q_sh;
  const __bf16* kp = static_cast<const __bf16*>(p.k) + it.b * p.k_sb + it.h * p.k_sh;
  const __bf16* vp = static_cast<const __bf16*>(p.v) + it.b * p.v_sb + it.h * p.v_sh;
  const int n_tiles = (p.Skv + kBN - 1) / kBN;

  // Q fragments (B operand of S^T = K Q^T): lane holds Q[qi][16 s + 8 hh .. +7].
  bf16x8 qf[8];
#pragma unroll
  for (int s = 0; s < 8; ++s)
    qf[s] = q_ok ? *reinterpret_cast<const bf16x8*>(qp + (int64_t)qi * p.q_ss + 16 * s + 8 * hh)
                 : bf16x8{};

  // Load streams: the wavefronts of group A stream K tiles into the K ring,
  // those of group B stream V tiles into the V ring; each issues its share
  // (LPW 1-KiB loads) at the start of its own Q-phase. A buffer resource
  // over the head's rows makes loads past the last key return zeros.
  const int wl = wave % (WAVES / 2);   // index inside the group
  const uint32_t k_rb = (uint32_t)(p.k_ss * 2), v_rb = (uint32_t)(p.v_ss * 2);
  const uint32_t my_rb = grp_b ? v_rb : k_rb;
  const void* my_src = grp_b ? (const void*)vp : (const void*)kp;
  const int my_rec = (int)((uint32_t)(p.Skv - 1) * my_rb + kD * 2);
  // Load j of this wavefront fills tile rows 4 (wl LPW + j) .. +3; lane l
  // fills LDS chunk l%16 of its row, which holds the row's global chunk
  // (l%16) ^ swizzle(row).
  uint32_t loff[LPW];
#pragma unroll
  for (int j = 0; j < LPW; ++j) {
    const int r = 4 * (wl * LPW + j) + (lane >> 4);
    const int pos = lane & 15;
    const int chunk = grp_b ? swz_v(r, pos) : swz_k(r, pos);
    loff[j] = (uint32_t)r * my_rb + ((uint32_t)chunk << 4);
  }
  unsigned char* my_ring = grp_b ? &lds_v[0][0] : &lds_k[0][0];
  auto issue = [&](int t) __device__ {
    const __amdgpu_buffer_rsrc_t rsrc =
        __builtin_amdgcn_make_buffer_rsrc((void*)my_src, (short)0, my_rec, 0x00020000);
    const uint32_t base = (uint32_t)(t * kBN) * my_rb;
    unsigned char* dst = my_ring + (t % kStages) * kTileBytes + wl * LPW * 1024;
#pragma unroll
    for (int j = 0; j < LPW; ++j)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (LDS_AS void*)(dst + j * 1024), 16,
                                               (int)(loff[j] + base), 0, 0, 0);
  };

  const float c = p.scale_log2;
  f32x16 acc[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) acc[db] = f32x16{};
  float m_run = kNegInf;  // running max of raw scores (both halves agree)
  float l_run = 0.0f;     // this half's partial sum of exp2(s c - m c)

  // Per-lane LDS byte offsets inside a tile, computed once. K fragment
  // i = 2 s + kb reads row kb*32 + l32, head_dim 16 s + 8 hh .. +7; the row's
  // swizzle depends on l32 only, so kb adds a plain 8 KiB.
  uint32_t kofs[8];
#pragma unroll
  for (int s = 0; s < 8; ++s) kofs[s] = (uint32_t)(l32 * 256 + (swz_k(l32, 2 * s + hh) << 4));
  // V^T fragment i = (kb*2 + jj)*4 + db comes from two transposing reads:
  // lane (16 g + 4 e + a) points at key kb*32 + jj*16 + 8 part + 4 (g/2) + e,
  // columns 32 db + 16 (g%2) + 4 a, and receives 4 keys of column 32 db + l%32.
  // The swizzle of row kb*32 + jj*16 + r depends on r only, so (kb, jj) add
  // plain multiples of 4 KiB.
  const int tg = lane >> 4, te = (lane >> 2) & 3, ta = lane & 3;
  uint32_t vofs[2][4];
#pragma unroll
  for (int part = 0; part < 2; ++part)
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      const int row = 8 * part + 4 * (tg >> 1) + te;
      const int col = db * 32 + 16 * (tg & 1) + 4 * ta;
      vofs[part][db] = (uint32_t)(row * 256 + (swz_v(row, col >> 3) << 4) + (col & 7) * 2);
    }
  // LDS byte addresses of the two rings, hidden from constant folding so
  // that per-phase addresses stay "register base + small immediate" instead
  // of dozens of hoisted absolute addresses.
  uint32_t lds_k_addr = (uint32_t)(uintptr_t)(LDS_AS unsigned char*)&lds_k[0][0];
  uint32_t lds_v_addr = (uint32_t)(uintptr_t)(LDS_AS unsigned char*)&lds_v[0][0];
  asm volatile("" : "+s"(lds_k_addr));
  asm volatile("" : "+s"(lds_v_addr));
  auto k_addr = [&](int t) __device__ -> KAddr {
    KAddr r;
    const uint32_t base = lds_k_addr + (uint32_t)(t % kStages) * kTileBytes;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      uint32_t o = kofs[s];
      asm volatile("" : "+v"(o));   // recomputed per phase: nothing to hoist
      r.a[s] = o + base;
    }
    return r;
  };
  auto v_addr = [&](int t) __device__ -> VAddr {
    VAddr r;
    const uint32_t base = lds_v_addr + (uint32_t)(t % kStages) * kTileBytes;
#pragma unroll
    for (int part = 0; part < 2; ++part)
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        uint32_t o = vofs[part][db];
        asm volatile("" : "+v"(o));
        r.a[part][db] = o + base;
      }
    return r;
  };
  auto kread = [&](const KAddr& ka, int i) __device__ -> bf16x8 {
    return *(LDS_AS const bf16x8*)(uintptr_t)(ka.a[i >> 1] + (i & 1) * 8192);
  };
  auto vread = [&](const VAddr& va, int i) __device__ -> bf16x8 {
    const int db = i & 3, jj = (i >> 2) & 1, kb = i >> 3;
    const uint32_t off = (kb * 32 + jj * 16) * 256;
    const s16x4 w0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS s16x4*)(uintptr_t)(va.a[0][db] + off));
    const s16x4 w1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS s16x4*)(uintptr_t)(va.a[1][db] + off));
    const s16x8 w8 = __builtin_shufflevector(w0, w1, 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_bit_cast(bf16x8, w8);
  };

  f32x16 st[2];                   // S(t) of the current Q/P pair
  bf16x8 pf0[2][2], pf1[2][2];    // P(t) for even / odd t

  auto q_phase = [&](int t) __device__ {
    const KAddr kt = k_addr(t);
    bf16x8 kf[16];
    kf[0] = kread(kt, 0);
    kf[1] = kread(kt, 1);
    st[0] = f32x16{};
    st[1] = f32x16{};
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if (i + 2 < 16) kf[i + 2] = kread(kt, i + 2);
      st[i & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[i], qf[i >> 1], st[i & 1], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);   // keep reads two MFMAs ahead, no further
    }
  };

  // P-phase of tile t: P(t) into pc; O^T += V(t-1)^T P(t-1)^T from pp.
  auto p_phase = [&](const bool WITH_PV, int t, bf16x8 (&pc)[2][2], bf16x8 (&pp)[2][2]) {
    const VAddr vt = v_addr(t + kStages - 1);
    bf16x8 vf[16];
    if (WITH_PV) {
      vf[0] = vread(vt, 0);
      vf[1] = vread(vt, 1);
    }
    const int key0 = t * kBN;
    if (key0 + kBN > p.Skv) {   // ragged last tile: keys past Skv do not exist
#pragma unroll
      for (int e = 0; e < 32; ++e) {
        const int r = e & 15;
        const int key = key0 + (e >> 4) * 32 + 8 * (r >> 2) + 4 * hh + (r & 3);
        if (key >= p.Skv) st[e >> 4][r] = kNegInf;
      }
    }
    float mx = st[0][0];
#pragma unroll
    for (int e = 1; e < 32; ++e) mx = fmaxf(mx, st[e >> 4][e & 15]);
    mx = pair_max(mx);
    // lazy rescale: move the running max only on an increase above 2^8
    const bool need = (mx - m_run) * c > kRescaleLog2;
    const float m_new = need ? mx : m_run;
    const float alpha = need ? __builtin_amdgcn_exp2f((m_run - m_new) * c) : 1.0f;
    const bool any_need = wave_any(need);
    l_run *= alpha;
    m_run = m_new;
    const float mc = (m_run == kNegInf) ? 0.0f : m_run * c;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if (WITH_PV) {
        if (i + 2 < 16) vf[i + 2] = vread(vt, i + 2);
        const int db = i & 3, jj = (i >> 2) & 1, kb = i >> 3;
        acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[i], pp[kb][jj], acc[db], 0, 0, 0);
      }
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int e = 2 * i + q, kb = e >> 4, r = e & 15;
        const float x = __builtin_amdgcn_exp2f(__builtin_fmaf(st[kb][r], c, -mc));
        l_run += x;
        pc[kb][r >> 3][r & 7] = (__bf16)x;
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    if (any_need) {
#pragma unroll
      for (int db = 0; db < 4; ++db) acc[db] *= alpha;
    }
  };

  // ---- prologue: group A loads K0 and K1, group B loads V0; all land
  // before interval 0.
  if (!grp_b) {
    issue(0);
    if (n_tiles > 1) issue(1);
  } else {
    issue(0);
  }
  wait_vmcnt<0>();
  barrier_no_fence();

  // ---- intervals. A wavefront's program is Q(0) P(0) Q(1) P(1) ... Q(n-1)
  // P(n-1) [ ] P(n), where P(n) runs on a tile past the end (every score
  // masked, so P(n) = 0) and only adds V(n-1)^T P(n-1)^T. Group A starts at
  // interval 0, group B one interval later; both meet every barrier. In its
  // Q-phase t (interval 2t for A, 2t+1 for B) a wavefront issues tile t + 2
  // of K (group A) or tile t + 1 of V (group B): K(t) lands by interval 2t,
  // V(t) by interval 2t + 1, two intervals after issue. Before each barrier
  // a wavefront waits for its loads issued two or more intervals back.
  const int lead = grp_b ? 1 : 2;
  int since_issue = 2;   // intervals since this wavefront last issued loads
  auto q_interval = [&](int t) __device__ {
    const bool do_issue = t + lead < n_tiles;
    if (do_issue) issue(t + lead);
    if (t < n_tiles) q_phase(t);
    since_issue = do_issue ? 0 : since_issue + 1;
    if (since_issue == 0) wait_vmcnt<LPW>();
    else wait_vmcnt<0>();
    barrier_no_fence();
  };
  auto p_end = [&]() __device__ {
    ++since_issue;
    if (since_issue == 1) wait_vmcnt<LPW>();
    else wait_vmcnt<0>();
    barrier_no_fence();
  };

  if (grp_b) barrier_no_fence();   // B idles in interval 0
  q_interval(0);
  p_phase(false, 0, pf0, pf1);
  p_end();
  for (int t = 1; t <= n_tiles; t += 2) {
    q_interval(t);
    p_phase(true, t, pf1, pf0);
    p_end();
    if (t + 1 > n_tiles) break;
    q_interval(t + 1);
    p_phase(true, t + 1, pf0, pf1);
    p_end();
  }
  if (!grp_b) barrier_no_fence();  // A idles in the last interval

  // ---- epilogue: combine halves, normalise, write O and LSE
  const float l_tot = pair_sum(l_run);
  if (!q_ok) return;
  float* op = p.o + it.b * p.o_sb + it.h * p.o_sh + (int64_t)qi * p.o_ss;
  const bool empty = !(l_tot > 0.0f);
  const float inv_l = empty ? 0.0f : 1.0f / l_tot;
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const int d = db * 32 + 8 * g4 + 4 * hh;
      f32x4 o4;
#pragma unroll
      for (int i = 0; i < 4; ++i) o4[i] = acc[db][4 * g4 + i] * inv_l;
      *reinterpret_cast<f32x4*>(op + d) = o4;
    }
  if (hh == 0) {
    const float lse = empty ? kNegInf : m_run * p.scale + __logf(l_tot);
    p.lse[it.b * p.lse_sb + it.h * p.lse_sh + qi] = lse;
  }
}

// ------------------------------- bf16 dense, one wavefront per SIMD, pipelined
//
// Four wavefronts of 32 query rows each, one per SIMD. Each wavefront runs a
// software pipeline over the key tiles, so that its own instruction stream
// keeps the matrix core and the VALU busy together:
//   phase 1 of step t: S(t+1) = K(t+1) Q^T (16 MFMA), interleaved with the
//       exp2 of the already-scaled S(t) into x(t) (fp32) and P(t) (bf16);
//   phase 2 of step t: O^T += V(t)^T P(t)^T (16 MFMA), interleaved with the
//       row sum of x(t), the row max of S(t+1), the lazy-rescale decision and
//       the scaling s c - m c of S(t+1).
// Every query's arithmetic (product order, exp2 arguments, summation order,
// rescale points, bf16 rounding of P) is the one of the other bf16 kernels,
// so all of them give the same bits.
//
// K/V tiles go HBM -> LDS directly (buffer_load ... lds) into two slots per
// tensor. Each slot is its own LDS variable and every access names its slot
// at compile time (the step loop is unrolled by two), so the compiler can
// tell the LDS reads of one slot from the loads in flight into the other and
// does not make the reads wait for them. A step has two barriers: one after
// phase 1 (all wavefronts are done with K(t+1)), one after phase 2 (done
// with V(t)). Step t issues V(t+1) at its start, into the slot V(t-1) left,
// and K(t+3) after its middle barrier, into the slot K(t+1) left; each load
// has about one and a half steps to land, and a wavefront waits only for
// the loads the next phase reads.

constexpr int kSpWaves = 4;
constexpr int kSpBM = kSpWaves * kQW;   // 128 query rows per workgroup

template <bool SPARSE>
__global__ __launch_bounds__(kSpWaves * 64, 1) void attn_fwd_bf16_sp_kernel(AttnParams p) {
  constexpr int LPW = (kTileBytes / 1024) / kSpWaves;   // 1-KiB loads per wavefront per tensor
  static_assert(LPW * kSpWaves * 1024 == kTileBytes, "tile/threads mismatch");
  static_assert(!SPARSE || kSpBM == kMaskBlock, "a sparse workgroup covers one mask row");

  __shared__ __attribute__((aligned(1024))) unsigned char lds_k0[kTileBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char lds_k1[kTileBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char lds_v0[kTileBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char lds_v1[kTileBytes];
  extern __shared__ unsigned short kept_dyn[];   // sparse: kept key blocks of the mask row
  __shared__ int wave_cnt[kSpWaves];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hh = lane >> 5;

  // Dense: workgroups walk the items XCD by XCD. Sparse: in the given order
  // (most kept blocks first).
  int item;
  if constexpr (SPARSE) {
    item = p.order ? p.order[blockIdx.x] : (int)blockIdx.x;
  } else {
    item = xcd_remap(blockIdx.x, gridDim.x);
  }
  const Item it = decode_item(item, p.n_qblk, p.H);
  const int qi = it.qblk * kSpBM + wave * kQW + l32;
  const bool q_ok = qi < p.Sq;
  const __bf16* qp = static_cast<const __bf16*>(p.q) + it.b * p.q_sb + it.h * p.q_sh;
  const __bf16* kp = static_cast<const __bf16*>(p.k) + it.b * p.k_sb + it.h * p.k_sh;
  const __bf16* vp = static_cast<const __bf16*>(p.v) + it.b * p.v_sb + it.h * p.v_sh;

  // Key tiles: dense, 64-key tiles in order; sparse, the two 64-key halves
  // of every kept 128-key block in ascending order, without a half that lies
  // wholly past the last key. Either way only the last tile can be ragged.
  int n_tiles;
  if constexpr (SPARSE) {
    const uint8_t* mrow = p.mask + (((int64_t)it.b * p.H + it.h) * p.n_mqb + it.qblk) * p.n_mkb;
    const int n_kept = build_kept_list<kSpWaves * 64>(mrow, p.n_mkb, kept_dyn, wave_cnt);
    n_tiles = 2 * n_kept;
    if (n_kept > 0 && (int)kept_dyn[n_kept - 1] * kMaskBlock + kBN >= p.Skv) n_tiles -= 1;
  } else {
    n_tiles = (p.Skv + kBN - 1) / kBN;
  }
  auto key0_of = [&](int t) __device__ -> int { return tile_key0<SPARSE>(t, kept_dyn); };

  // Q fragments (B operand of S^T = K Q^T): lane holds Q[qi][16 s + 8 hh .. +7].
  bf16x8 qf[8];
#pragma unroll
  for (int s = 0; s < 8; ++s)
    qf[s] = q_ok ? *reinterpret_cast<const bf16x8*>(qp + (int64_t)qi * p.q_ss + 16 * s + 8 * hh)
                 : bf16x8{};

  // ---- tile loads: every wavefront issues LPW 1-KiB loads per tensor tile.
  // Load j of this wavefront fills tile rows 4 (wave LPW + j) .. +3; lane l
  // fills LDS chunk l%16 of its row, which holds the row's global chunk
  // (l%16) ^ swizzle(row). A buffer resource over the head's rows makes
  // loads past the last key return zeros.
  const uint32_t k_rb = (uint32_t)(p.k_ss * 2), v_rb = (uint32_t)(p.v_ss * 2);
  const int k_rec = (int)((uint32_t)(p.Skv - 1) * k_rb + kD * 2);
  const int v_rec = (int)((uint32_t)(p.Skv - 1) * v_rb + kD * 2);
  uint32_t koff[LPW], voff[LPW];
#pragma unroll
  for (int j = 0; j < LPW; ++j) {
    const int r = 4 * (wave * LPW + j) + (lane >> 4);
    const int pos = lane & 15;
    koff[j] = (uint32_t)r * k_rb + ((uint32_t)swz_k(r, pos) << 4);
    voff[j] = (uint32_t)r * v_rb + ((uint32_t)swz_v(r, pos) << 4);
  }
  auto kslot = [&](int slot) __device__ -> unsigned char* { return slot ? lds_k1 : lds_k0; };
  auto vslot = [&](int slot) __device__ -> unsigned char* { return slot ? lds_v1 : lds_v0; };
  auto issue_k = [&](int t) __device__ {
    const __amdgpu_buffer_rsrc_t rsrc =
        __builtin_amdgcn_make_buffer_rsrc((void*)kp, (short)0, k_rec, 0x00020000);
    const uint32_t base = (uint32_t)key0_of(t) * k_rb;
    unsigned char* dst = kslot(t & 1) + wave * LPW * 1024;
#pragma unroll
    for (int j = 0; j < LPW; ++j)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (LDS_AS void*)(dst + j * 1024), 16,
                                               (int)(koff[j] + base), 0, 0, 0);
  };
  auto issue_v = [&](int t) __device__ {
    const __amdgpu_buffer_rsrc_t rsrc =
        __builtin_amdgcn_make_buffer_rsrc((void*)vp, (short)0, v_rec, 0x00020000);
    const uint32_t base = (uint32_t)key0_of(t) * v_rb;
    unsigned char* dst = vslot(t & 1) + wave * LPW * 1024;
#pragma unroll
    for (int j = 0; j < LPW; ++j)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (LDS_AS void*)(dst + j * 1024), 16,
                                               (int)(voff[j] + base), 0, 0, 0);
  };

  // ---- LDS fragment offsets inside a tile (per lane, loop-invariant). K
  // fragment i = 2 s + kb reads row kb*32 + l32, head_dim 16 s + 8 hh .. +7.
  // V^T fragment i = (kb*2 + jj)*4 + db comes from two transposing reads:
  // lane (16 g + 4 e + a) points at key kb*32 + jj*16 + 8 part + 4 (g/2) + e,
  // columns 32 db + 16 (g%2) + 4 a, and receives 4 keys of column 32 db + l%32.
  uint32_t kofs[8];
#pragma unroll
  for (int s = 0; s < 8; ++s) kofs[s] = (uint32_t)(l32 * 256 + (swz_k(l32, 2 * s + hh) << 4));
  const int tg = lane >> 4, te = (lane >> 2) & 3, ta = lane & 3;
  uint32_t vofs[2][4];
#pragma unroll
  for (int part = 0; part < 2; ++part)
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      const int row = 8 * part + 4 * (tg >> 1) + te;
      const int col = db * 32 + 16 * (tg & 1) + 4 * ta;
      vofs[part][db] = (uint32_t)(row * 256 + (swz_v(row, col >> 3) << 4) + (col & 7) * 2);
    }
  auto kread = [&](int slot, int i) __device__ -> bf16x8 {
    const LDS_AS unsigned char* b = (LDS_AS const unsigned char*)kslot(slot);
    return *(LDS_AS const bf16x8*)(b + kofs[i >> 1] + (i & 1) * 8192);
  };
  auto vread = [&](int slot, int i) __device__ -> bf16x8 {
    const int db = i & 3, jj = (i >> 2) & 1, kb = i >> 3;
    const LDS_AS unsigned char* b = (LDS_AS const unsigned char*)vslot(slot) + (kb * 32 + jj * 16) * 256;
    const s16x4 w0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS s16x4*)(b + vofs[0][db]));
    const s16x4 w1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS s16x4*)(b + vofs[1][db]));
    const s16x8 w8 = __builtin_shufflevector(w0, w1, 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_bit_cast(bf16x8, w8);
  };

  // ---- softmax state
  const float c = p.scale_log2;
  f32x16 acc[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) acc[db] = f32x16{};
  float m_run = kNegInf;   // running max of raw scores (both halves agree)
  float mc = 0.0f;         // m_run * c, or 0 while m_run = -inf
  float l_run = 0.0f;      // this half's partial sum of exp2(s c - m c)
  f32x16 sa[2], sb[2];     // S of two consecutive tiles: st[kb][r]
  bf16x8 pf[2][2];         // P(t): pf[kb][jj]

  // Row max of the raw scores st -> lazy-rescale decision -> st becomes
  // s c - m c. Split into 16 slices that phase 2 spreads over its 16 MFMAs:
  // slices 0-7 take the max of scores 4k .. 4k+3, slice 8 decides, slices
  // 9-15 scale five scores each.
  float part_max = kNegInf, alpha = 1.0f;
  bool any_need = false;
  auto softmax_slice = [&](f32x16 (&st)[2], int k) __device__ {
    if (k < 8) {
#pragma unroll
      for (int e = 4 * k; e < 4 * k + 4; ++e) part_max = fmaxf(part_max, st[e >> 4][e & 15]);
    } else if (k == 8) {
      const float mx = pair_max(part_max);
      part_max = kNegInf;
      const bool need = (mx - m_run) * c > kRescaleLog2;
      const float m_new = need ? mx : m_run;
      alpha = need ? __builtin_amdgcn_exp2f((m_run - m_new) * c) : 1.0f;
      any_need = wave_any(need);
      m_run = m_new;
      mc = (m_run == kNegInf) ? 0.0f : m_run * c;
    } else {
      const int e0 = 5 * (k - 9), e1 = e0 + 5 < 32 ? e0 + 5 : 32;
#pragma unroll
      for (int e = e0; e < e1; ++e) {
        float y = __builtin_fmaf(st[e >> 4][e & 15], c, -mc);
        asm volatile("" : "+v"(y));   // computed here, not sunk into the next step
        st[e >> 4][e & 15] = y;
      }
    }
  };
  auto mask_tile = [&](f32x16 (&st)[2], int key0) __device__ {
    if (key0 + kBN > p.Skv) {
      const int lim = p.Skv - key0 - 4 * hh;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int off = 8 * (r >> 2) + (r & 3);
        if (off >= lim) st[0][r] = kNegInf;
        if (off + 32 >= lim) st[1][r] = kNegInf;
      }
    }
  };

  // phase 1 of step t: S(t+1) -> sn (if DO_QK), interleaved with
  // x(t) = exp2(sc) kept in sc and P(t) = bf16(x(t)) in pf
  auto phase1 = [&](const bool DO_QK, int t, f32x16 (&sc)[2], f32x16 (&sn)[2]) __device__ {
    const int ks = (t + 1) & 1;
    bf16x8 kf[16];
    if (DO_QK) {
      kf[0] = kread(ks, 0);
      kf[1] = kread(ks, 1);
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if (DO_QK) {
        if (i + 2 < 16) kf[i + 2] = kread(ks, i + 2);
        if (i < 2)
          sn[i & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[i], qf[i >> 1], f32x16{}, 0, 0, 0);
        else
          sn[i & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[i], qf[i >> 1], sn[i & 1], 0, 0, 0);
      }
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int e = 2 * i + q, kb = e >> 4, r = e & 15;
        const float x = __builtin_amdgcn_exp2f(sc[kb][r]);
        asm volatile("" ::"v"(x));   // computed here, next to this MFMA
        sc[kb][r] = x;
        pf[kb][r >> 3][r & 7] = (__bf16)x;
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // phase 2 of step t: O^T += V(t)^T P(t)^T, interleaved with l += x(t) and
  // (if HAS_NEXT) the softmax slices of S(t+1)
  auto phase2 = [&](const bool HAS_NEXT, const bool MAYBE_RAGGED, int t, f32x16 (&sc)[2],
                    f32x16 (&sn)[2]) __device__ {
    if (HAS_NEXT && MAYBE_RAGGED) mask_tile(sn, key0_of(t + 1));
    const int vs = t & 1;
    bf16x8 vf[16];
    vf[0] = vread(vs, 0);
    vf[1] = vread(vs, 1);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if (i + 2 < 16) vf[i + 2] = vread(vs, i + 2);
      const int db = i & 3, jj = (i >> 2) & 1, kb = i >> 3;
      acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[i], pf[kb][jj], acc[db], 0, 0, 0);
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int e = 2 * i + q;
        float l = l_run + sc[e >> 4][e & 15];
        asm volatile("" : "+v"(l));   // summed here, in key order
        l_run = l;
      }
      if (HAS_NEXT) softmax_slice(sn, i);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (HAS_NEXT) {
      l_run *= alpha;
      if (any_need) {
#pragma unroll
        for (int db = 0; db < 4; ++db) acc[db] *= alpha;
      }
    }
  };

  // waits until at most n (0, LPW or 2 LPW) of this wavefront's loads are
  // still in flight
  auto wait_le = [&](int n) __device__ {
    if (n == 0) wait_vmcnt<0>();
    else if (n == LPW) wait_vmcnt<LPW>();
    else wait_vmcnt<2 * LPW>();
  };

  // A sparse row without kept blocks attends to no key: it skips straight
  // to the epilogue, which writes O = 0 and LSE = -inf.
  if (n_tiles > 0) {
    // ---- prologue: K0, K1 and V0 in flight; S(0), its max, the rescale
    // decision and its scaling once K0 landed; then K1 must have landed and
    // K2 goes into K0's slot.
    issue_k(0);
    if (n_tiles > 1) issue_k(1);
    issue_v(0);
    wait_le(n_tiles > 1 ? 2 * LPW : LPW);
    barrier_no_fence();
    {
      sa[0] = f32x16{};
      sa[1] = f32x16{};
#pragma unroll
      for (int i = 0; i < 16; ++i)
        sa[i & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kread(0, i), qf[i >> 1], sa[i & 1], 0, 0, 0);
      mask_tile(sa, key0_of(0));
#pragma unroll
      for (int k = 0; k < 16; ++k) softmax_slice(sa, k);
      l_run *= alpha;   // l_run = 0: the product stays 0
    }
    wait_le(LPW);   // K1 (V0 may stay in flight)
    barrier_no_fence();
    if (n_tiles > 2) issue_k(2);

    // one step: tile t's scaled scores in sc, S(t+1) into sn (if HAS_NEXT,
    // i.e. t + 1 < n_tiles)
    auto step = [&](const bool HAS_NEXT, const bool MAYBE_RAGGED, int t, f32x16 (&sc)[2],
                    f32x16 (&sn)[2]) __device__ {
      if (HAS_NEXT) issue_v(t + 1);
      phase1(HAS_NEXT, t, sc, sn);
      // V(t) next; in flight after it: K(t+2), V(t+1)
      wait_le((t + 2 < n_tiles ? LPW : 0) + (HAS_NEXT ? LPW : 0));
      barrier_no_fence();
      if (t + 3 < n_tiles) issue_k(t + 3);
      phase2(HAS_NEXT, MAYBE_RAGGED, t, sc, sn);
      if (t + 2 < n_tiles) {
        // K(t+2) next; in flight after it: V(t+1), K(t+3)
        wait_le((HAS_NEXT ? LPW : 0) + (t + 3 < n_tiles ? LPW : 0));
        barrier_no_fence();
      }
    };

    // t is even at the top of the loop, so every slot index above is a
    // compile-time constant. Tiles before the last one are never ragged: the
    // loop runs steps whose next tile is at most n_tiles - 2.
    int t = 0;
    for (; t + 3 < n_tiles; t += 2) {
      step(true, false, t, sa, sb);
      step(true, false, t + 1, sb, sa);
    }
    const int rest = n_tiles - t;   // 1, 2 or 3
    if (rest == 3) {
      step(true, false, t, sa, sb);
      step(true, true, t + 1, sb, sa);
      step(false, false, t + 2, sa, sa);
    } else if (rest == 2) {
      step(true, true, t, sa, sb);
      step(false, false, t + 1, sb, sb);
    } else {
      step(false, false, t, sa, sa);
    }
  }   // n_tiles > 0

  // ---- epilogue: combine halves, normalise, write O and LSE
  const float l_tot = pair_sum(l_run);
  if (!q_ok) return;
  float* op = p.o + it.b * p.o_sb + it.h * p.o_sh + (int64_t)qi * p.o_ss;
  const bool empty = !(l_tot > 0.0f);
  const float inv_l = empty ? 0.0f : 1.0f / l_tot;
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const int d = db * 32 + 8 * g4 + 4 * hh;
      f32x4 o4;
#pragma unroll
      for (int i = 0; i < 4; ++i) o4[i] = acc[db][4 * g4 + i] * inv_l;
      *reinterpret_cast<f32x4*>(op + d) = o4;
    }
  if (hh == 0) {
    const float lse = empty ? kNegInf : m_run * p.scale + __logf(l_tot);
    p.lse[it.b * p.lse_sb + it.h * p.lse_sh + qi] = lse;
  }
}

// ------------------------------------------------------------------ f32 path

// LDS row stride (floats) of the fp32 tiles: padded against bank conflicts.
constexpr int kF32Row = kD + 4;

template <int WAVES, bool SPARSE>
__global__ __launch_bounds__(WAVES * 64) void attn_fwd_f32_kernel(AttnParams p) {
  constexpr int NT = WAVES * 64;
  constexpr int BM = WAVES * kQW;
  static_assert(!SPARSE || BM == kMaskBlock, "sparse kernel works on one mask row");

  __shared__ __attribute__((aligned(16))) float lds_k[kBN * kF32Row];
  __shared__ __attribute__((aligned(16))) float lds_v[kBN * kF32Row];
  extern __shared__ unsigned short kept_dyn[];
  __shared__ int wave_cnt[WAVES];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int l32 = lane & 31, hh = lane >> 5;

  int item;
  if constexpr (SPARSE) {
    item = p.order ? p.order[blockIdx.x] : (int)blockIdx.x;
  } else {
    item = xcd_remap(blockIdx.x, gridDim.x);
  }
  const Item it = decode_item(item, p.n_qblk, p.H);
  const int qi = it.qblk * BM + wave * kQW + l32;
  const bool q_ok = qi < p.Sq;

  const float* qp = static_cast<const float*>(p.q) + it.b * p.q_sb + it.h * p.q_sh;
  const float* kp = static_cast<const float*>(p.k) + it.b * p.k_sb + it.h * p.k_sh;
  const float* vp = static_cast<const float*>(p.v) + it.b * p.v_sb + it.h * p.v_sh;

  int n_tiles;
  const unsigned short* kept = kept_dyn;
  if constexpr (SPARSE) {
    const uint8_t* mrow = p.mask + (((int64_t)it.b * p.H + it.h) * p.n_mqb + it.qblk) * p.n_mkb;
    n_tiles = 2 * build_kept_list<NT>(mrow, p.n_mkb, kept_dyn, wave_cnt);
  } else {
    n_tiles = (p.Skv + kBN - 1) / kBN;
  }

  // Q: lane holds Q[qi][2 s + hh], s = 0..63
  float qf[64];
#pragma unroll
  for (int s = 0; s < 64; ++s) qf[s] = q_ok ? qp[(int64_t)qi * p.q_ss + 2 * s + hh] : 0.0f;

  f32x16 acc[4];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[db][r] = 0.0f;
  float m_run = kNegInf, l_run = 0.0f;
  const float c = p.scale_log2;

  for (int t = 0; t < n_tiles; ++t) {
    const int key0 = tile_key0<SPARSE>(t, kept);
    // stage the tile: 64 rows x 32 float4 chunks per tensor
    for (int cid = tid; cid < kBN * (kD / 4); cid += NT) {
      const int row = cid >> 5, ch = cid & 31;
      const int key = key0 + row;
      f32x4 kv = {0.f, 0.f, 0.f, 0.f}, vv = {0.f, 0.f, 0.f, 0.f};
      if (key < p.Skv) {
        kv = *reinterpret_cast<const f32x4*>(kp + (int64_t)key * p.k_ss + ch * 4);
        vv = *reinterpret_cast<const f32x4*>(vp + (int64_t)key * p.v_ss + ch * 4);
      }
      *reinterpret_cast<f32x4*>(&lds_k[row * kF32Row + ch * 4]) = kv;
      *reinterpret_cast<f32x4*>(&lds_v[row * kF32Row + ch * 4]) = vv;
    }
    __syncthreads();

    f32x16 st[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) st[kb][r] = 0.0f;
      const int row = kb * 32 + l32;
#pragma unroll
      for (int s = 0; s < 64; ++s)
        st[kb] = __builtin_amdgcn_mfma_f32_32x32x2f32(lds_k[row * kF32Row + 2 * s + hh], qf[s],
                                                      st[kb], 0, 0, 0);
    }
    if (key0 + kBN > p.Skv) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = key0 + kb * 32 + 8 * (r >> 2) + 4 * hh + (r & 3);
          if (key >= p.Skv) st[kb][r] = kNegInf;
        }
    }
    float mx = st[0][0];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, st[kb][r]);
    mx = pair_max(mx);
    const bool need = (mx - m_run) * c > kRescaleLog2;
    if (wave_any(need)) {
      const float m_new = need ? mx : m_run;
      const float alpha = need ? __builtin_amdgcn_exp2f((m_run - m_new) * c) : 1.0f;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[db][r] *= alpha;
      l_run *= alpha;
      m_run = m_new;
    }
    const float mc = (m_run == kNegInf) ? 0.0f : m_run * c;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(st[kb][r], c, -mc));
        l_run += e;
        st[kb][r] = e;
      }
    // O^T += V^T P^T, one key per MFMA step: half hh uses key
    // kb*32 + 8 (r/4) + 4 hh + r%4, the key its register r holds.
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = kb * 32 + 8 * (r >> 2) + 4 * hh + (r & 3);
#pragma unroll
        for (int db = 0; db < 4; ++db)
          acc[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(lds_v[row * kF32Row + db * 32 + l32],
                                                         st[kb][r], acc[db], 0, 0, 0);
      }
    __syncthreads();
  }

  const float l_tot = pair_sum(l_run);
  if (!q_ok) return;
  float* op = p.o + it.b * p.o_sb + it.h * p.o_sh + (int64_t)qi * p.o_ss;
  const bool empty = !(l_tot > 0.0f);
  const float inv_l = empty ? 0.0f : 1.0f / l_tot;
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const int d = db * 32 + 8 * g4 + 4 * hh;
      f32x4 o4;
#pragma unroll
      for (int i = 0; i < 4; ++i) o4[i] = acc[db][4 * g4 + i] * inv_l;
      *reinterpret_cast<f32x4*>(op + d) = o4;
    }
  if (hh == 0) {
    const float lse = empty ? kNegInf : m_run * p.scale + __logf(l_tot);
    p.lse[it.b * p.lse_sb + it.h * p.lse_sh + qi] = lse;
  }
}

// O = 0, LSE = -inf for every row (attention over an empty key set).
__global__ void attn_empty_kernel(AttnParams p) {
  const int64_t rows = (int64_t)p.B * p.Sq * p.H;
  for (int64_t r = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; r < rows;
       r += (int64_t)gridDim.x * blockDim.x) {
    const int h = (int)(r % p.H);
    const int64_t bs = r / p.H;
    const int s = (int)(bs % p.Sq);
    const int b = (int)(bs / p.Sq);
    float* op = p.o + b * p.o_sb + h * p.o_sh + (int64_t)s * p.o_ss;
    for (int d = 0; d < kD; d += 4) *reinterpret_cast<f32x4*>(op + d) = f32x4{0.f, 0.f, 0.f, 0.f};
    p.lse[b * p.lse_sb + h * p.lse_sh + s] = kNegInf;
  }
}

}  // namespace

hipError_t launch_attn_dense(const AttnParams& p0, DType dt, hipStream_t s) {
  AttnParams p = p0;
  if (dt == DType::F32) {
    p.n_qblk = (p.Sq + 127) / 128;
    p.n_items = p.B * p.H * p.n_qblk;
    hipLaunchKernelGGL((attn_fwd_f32_kernel<4, false>), dim3(p.n_items), dim3(256), 0, s, p);
    return hipGetLastError();
  }
  // Grids of at least two 256-row workgroups per CU run the ping-pong
  // kernel; smaller ones the one-wavefront-per-SIMD kernel, which keeps every
  // SIMD busy with a single 128-row workgroup per CU. Both give the same bits.
  const int64_t items_pp = (int64_t)p.B * p.H * ((p.Sq + 255) / 256);
  if (items_pp >= 512) {
    p.n_qblk = (p.Sq + 255) / 256;
    p.n_items = p.B * p.H * p.n_qblk;
    hipLaunchKernelGGL((attn_fwd_bf16_pp_kernel<8>), dim3(p.n_items), dim3(512), 0, s, p);
  } else {
    p.n_qblk = (p.Sq + kSpBM - 1) / kSpBM;
    p.n_items = p.B * p.H * p.n_qblk;
    hipLaunchKernelGGL(attn_fwd_bf16_sp_kernel<false>, dim3(p.n_items), dim3(kSpWaves * 64), 0, s, p);
  }
  return hipGetLastError();
}

hipError_t launch_attn_sparse(const AttnParams& p0, DType dt, hipStream_t s) {
  AttnParams p = p0;
  p.n_qblk = p.n_mqb;
  p.n_items = p.B * p.H * p.n_mqb;
  const size_t dyn = sizeof(unsigned short) * (size_t)p.n_mkb;
  if (dt == DType::F32)
    hipLaunchKernelGGL((attn_fwd_f32_kernel<4, true>), dim3(p.n_items), dim3(256), dyn, s, p);
  else
    hipLaunchKernelGGL(attn_fwd_bf16_sp_kernel<true>, dim3(p.n_items), dim3(kSpWaves * 64), dyn, s, p);
  return hipGetLastError();
}

hipError_t launch_attn_empty(const AttnParams& p, hipStream_t s) {
  const int64_t rows = (int64_t)p.B * p.Sq * p.H;
  int64_t blocks = (rows + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(attn_empty_kernel, dim3((unsigned)blocks), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace lsh
