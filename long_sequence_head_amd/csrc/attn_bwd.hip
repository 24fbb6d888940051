// Attention backward for gfx950: dQ, dK, dV of dense softmax attention from
// bf16 Q, K, V, the upstream gradient dO and the forward's float32 O and
// LSE. With P = exp(scale Q K^T - LSE) (the forward's softmax, rebuilt from
// its log-sum-exp) the gradients are
//   dV = P^T dO,  dP = dO V^T,  Delta = rowsum(dO * O) = rowsum(P * dP),
//   dS = P * (dP - Delta),  dQ = scale dS K,  dK = scale dS^T Q
// (the derivative of the forward of "LLM Lab Notes 05: Attention Tensor
// Parallelism", sections 2-3; the backward pass is the one whose speed-ups
// the CHARM+ page reports under "Measured Speedups").
//
// Three kernels, no atomics, so repeated runs give the same bits:
//  * rows:  LSE * log2(e) and Delta of every query row, into a workspace
//           laid out in 64-row tiles; rows past Sq get LSE = +inf and
//           Delta = 0, so their P and dS are exactly 0.
//  * dK/dV: a workgroup owns 128 keys (32 per wavefront; the wavefront
//           keeps K and V of its keys in registers) and streams every
//           64-row query tile of the head through LDS. Per 32 queries:
//           S = Q K^T and dP = dO V^T with keys in lanes, P and dS in
//           registers, then dV^T += dO^T P and dK^T += Q^T dS.
//  * dQ:    a workgroup owns 128 queries (Q and dO in registers) and
//           streams 64-key tiles: S^T = K Q^T and dP^T = V dO^T with
//           queries in lanes, then dQ^T += K^T dS^T.
// S and dP are formed in both passes: 14 units of matrix work for the 10 of
// the definition, in exchange for determinism without atomics and without a
// quadratic dS buffer.
//
// Both streaming kernels run one wavefront per SIMD and keep three LDS slots
// per streamed tensor: step t issues the loads of tile t + 2 into the slot
// tile t - 1 left, computes tile t, then waits for tile t + 1 and meets the
// other wavefronts at one barrier. Each load has two steps to land.
#include "attn_common.hpp"

namespace lsh {
namespace {

constexpr int kBwdWaves = 4;
constexpr int kBwdBlk = kBwdWaves * 32;      // keys (dK/dV) or queries (dQ) per workgroup
constexpr int kAuxRow = 2 * kBwdQT;          // floats of one aux tile
constexpr int kAuxBytes = kAuxRow * 4;
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ f32x16 mfma16(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// ------------------------------------------------------------- row statistics
// 16 lanes per query row: lane sub multiplies head_dim 8 sub .. 8 sub + 7,
// then a butterfly over the 16 lanes sums them in a fixed order.
__global__ __launch_bounds__(256) void attn_bwd_rows_kernel(BwdParams p) {
  const int rows = p.n_qt * kBwdQT;
  const int64_t gid = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);
  const int sub = threadIdx.x & 15;
  const int bh = (int)(gid / rows), i = (int)(gid % rows);
  const int b = bh / p.H, h = bh % p.H;
  float acc = 0.0f;
  if (i < p.Sq) {
    const __bf16* dop = static_cast<const __bf16*>(p.dout) + b * p.do_sb + h * p.do_sh +
                        (int64_t)i * p.do_ss + 8 * sub;
    const float* op = p.o + b * p.o_sb + h * p.o_sh + (int64_t)i * p.o_ss + 8 * sub;
    const bf16x8 d8 = *reinterpret_cast<const bf16x8*>(dop);
    const f32x4 o0 = *reinterpret_cast<const f32x4*>(op);
    const f32x4 o1 = *reinterpret_cast<const f32x4*>(op + 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) acc = __builtin_fmaf((float)d8[e], o0[e], acc);
#pragma unroll
    for (int e = 0; e < 4; ++e) acc = __builtin_fmaf((float)d8[4 + e], o1[e], acc);
  }
#pragma unroll
  for (int m = 1; m < 16; m <<= 1) acc += __shfl_xor(acc, m, 16);
  if (sub == 0) {
    float* a = p.aux + ((int64_t)bh * p.n_qt + i / kBwdQT) * kAuxRow + (i % kBwdQT);
    a[0] = i < p.Sq ? p.lse[b * p.lse_sb + h * p.lse_sh + i] * kLog2e : __builtin_inff();
    a[kBwdQT] = acc;
  }
}

// --------------------------------------------------------------------- dK, dV
__global__ __launch_bounds__(kBwdWaves * 64, 1) void attn_bwd_dkdv_kernel(BwdParams p) {
  constexpr int LPW = (kTileBytes / 1024) / kBwdWaves;   // 1-KiB loads per wavefront per tensor
  constexpr int LOADS = 2 * LPW + 1;                     // + one for the aux tile
  static_assert(LPW * kBwdWaves * 1024 == kTileBytes, "tile/threads mismatch");
  static_assert(kBwdQT == kBN, "query tiles have the shape of key tiles");

  __shared__ __attribute__((aligned(1024))) unsigned char lq0[kTileBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char lq1[kTileBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char lq2[kTileBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char ld0[kTileBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char ld1[kTileBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char ld2[kTileBytes];
  __shared__ __attribute__((aligned(512))) unsigned char la0[kAuxBytes];
  __shared__ __attribute__((aligned(512))) unsigned char la1[kAuxBytes];
  __shared__ __attribute__((aligned(512))) unsigned char la2[kAuxBytes];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hh = lane >> 5;

  const int n_kblk = (p.Skv + kBwdBlk - 1) / kBwdBlk;
  const int item = xcd_remap(blockIdx.x, gridDim.x);
  const int kblk = item % n_kblk, bh = item / n_kblk;
  const int h = bh % p.H, b = bh / p.H;
  const int kj = kblk * kBwdBlk + wave * 32 + l32;
  const bool k_ok = kj < p.Skv;
  const __bf16* qp = static_cast<const __bf16*>(p.q) + b * p.q_sb + h * p.q_sh;
  const __bf16* kp = static_cast<const __bf16*>(p.k) + b * p.k_sb + h * p.k_sh;
  const __bf16* vp = static_cast<const __bf16*>(p.v) + b * p.v_sb + h * p.v_sh;
  const __bf16* dop = static_cast<const __bf16*>(p.dout) + b * p.do_sb + h * p.do_sh;

  // K and V of this lane's key: the B operands of S = Q K^T and dP = dO V^T
  // (lane holds head_dim 16 s + 8 hh .. +7 of key kj). Keys past Skv are 0.
  bf16x8 kf[8], vf[8];
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    kf[s] = k_ok ? *reinterpret_cast<const bf16x8*>(kp + (int64_t)kj * p.k_ss + 16 * s + 8 * hh)
                 : bf16x8{};
    vf[s] = k_ok ? *reinterpret_cast<const bf16x8*>(vp + (int64_t)kj * p.v_ss + 16 * s + 8 * hh)
                 : bf16x8{};
  }

  // ---- tile loads (Q and dO rows with the swz_v swizzle; rows past Sq
  // read as zeros) and the aux tile (each wavefront loads 128 of its bytes)
  const uint32_t q_rb = (uint32_t)(p.q_ss * 2), do_rb = (uint32_t)(p.do_ss * 2);
  const int q_rec = (int)((uint32_t)(p.Sq - 1) * q_rb + kD * 2);
  const int do_rec = (int)((uint32_t)(p.Sq - 1) * do_rb + kD * 2);
  uint32_t qoff[LPW], dooff[LPW];
#pragma unroll
  for (int j = 0; j < LPW; ++j) {
    const int r = 4 * (wave * LPW + j) + (lane >> 4);
    const uint32_t c16 = (uint32_t)swz_v(r, lane & 15) << 4;
    qoff[j] = (uint32_t)r * q_rb + c16;
    dooff[j] = (uint32_t)r * do_rb + c16;
  }
  const i32x4 q_rsrc = make_rsrc(qp, q_rec), do_rsrc = make_rsrc(dop, do_rec);
  const i32x4 a_rsrc = make_rsrc(p.aux + (int64_t)bh * p.n_qt * kAuxRow, p.n_qt * kAuxBytes);
  auto qslot = [&](int s) __device__ -> unsigned char* { return s == 0 ? lq0 : s == 1 ? lq1 : lq2; };
  auto dslot = [&](int s) __device__ -> unsigned char* { return s == 0 ? ld0 : s == 1 ? ld1 : ld2; };
  auto aslot = [&](int s) __device__ -> unsigned char* { return s == 0 ? la0 : s == 1 ? la1 : la2; };
  auto issue = [&](int t, int s) __device__ {
    const uint32_t bq = (uint32_t)t * kBwdQT * q_rb, bd = (uint32_t)t * kBwdQT * do_rb;
    const uint32_t dst_q = lds_addr(qslot(s)) + wave * LPW * 1024;
    const uint32_t dst_d = lds_addr(dslot(s)) + wave * LPW * 1024;
#pragma unroll
    for (int j = 0; j < LPW; ++j) lds_dma16(dst_q + j * 1024, qoff[j] + bq, q_rsrc);
#pragma unroll
    for (int j = 0; j < LPW; ++j) lds_dma16(dst_d + j * 1024, dooff[j] + bd, do_rsrc);
    if (lane < 8)
      lds_dma16(lds_addr(aslot(s)) + wave * 128, (uint32_t)t * kAuxBytes + wave * 128 + lane * 16,
                a_rsrc);
  };

  // ---- LDS read offsets: row fragment s of a 32-row block reads row l32,
  // head_dim 16 s + 8 hh .. +7 (A operand of S and dP); tr_read gives the
  // transposed fragments (A operands of dV^T and dK^T).
  uint32_t rofs[8];
#pragma unroll
  for (int s = 0; s < 8; ++s) rofs[s] = (uint32_t)(l32 * 256 + (swz_v(l32, 2 * s + hh) << 4));
  uint32_t tofs[2][4];
  tr_offsets(lane, tofs);

  const float c = p.scale_log2;
  f32x16 acc_dv[4], acc_dk[4];   // dV^T, dK^T: [head_dim][key], key = lane
#pragma unroll
  for (int db = 0; db < 4; ++db) {
    acc_dv[db] = f32x16{};
    acc_dk[db] = f32x16{};
  }

  auto compute = [&](int s) __device__ {
    const unsigned char* tq = qslot(s);
    const unsigned char* td = dslot(s);
    const LDS_AS unsigned char* lq = (LDS_AS const unsigned char*)tq;
    const LDS_AS unsigned char* ld = (LDS_AS const unsigned char*)td;
    const LDS_AS unsigned char* la = (LDS_AS const unsigned char*)aslot(s);
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      // S and dP of queries 32 qb + 8 (r / 4) + 4 hh + r % 4 (register r)
      // and this lane's key
      f32x16 sc = f32x16{}, dp = f32x16{};
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const bf16x8 aq = *(LDS_AS const bf16x8*)(lq + qb * 8192 + rofs[i]);
        const bf16x8 ad = *(LDS_AS const bf16x8*)(ld + qb * 8192 + rofs[i]);
        sc = mfma16(aq, kf[i], sc);
        dp = mfma16(ad, vf[i], dp);
      }
      // P = exp2(S c - LSE log2 e), dS = P (dP - Delta), packed in the order
      // tr_read expects
      bf16x8 pp[2], pds[2];
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int row = 32 * qb + 8 * g + 4 * hh;
        const f32x4 l4 = *(LDS_AS const f32x4*)(la + row * 4);
        const f32x4 d4 = *(LDS_AS const f32x4*)(la + kBwdQT * 4 + row * 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * g + e;
          const float pr = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[r], c, -l4[e]));
          const float ds = pr * (dp[r] - d4[e]);
          pp[r >> 3][r & 7] = (__bf16)pr;
          pds[r >> 3][r & 7] = (__bf16)ds;
        }
      }
#pragma unroll
      for (int jj = 0; jj < 2; ++jj)
#pragma unroll
        for (int db = 0; db < 4; ++db) {
          const int i = (qb * 2 + jj) * 4 + db;
          acc_dv[db] = mfma16(tr_read(td, tofs, i), pp[jj], acc_dv[db]);
          acc_dk[db] = mfma16(tr_read(tq, tofs, i), pds[jj], acc_dk[db]);
        }
    }
  };

  const int n_t = p.n_qt;
  auto step = [&](int s, int t) __device__ {
    if (t + 2 < n_t) issue(t + 2, (s + 2) % 3);
    compute(s);
    if (t + 1 < n_t) {
      if (t + 2 < n_t) wait_vmcnt<LOADS>();
      else wait_vmcnt<0>();
      barrier_no_fence();
    }
  };
  issue(0, 0);
  if (n_t > 1) {
    issue(1, 1);
    wait_vmcnt<LOADS>();
  } else {
    wait_vmcnt<0>();
  }
  barrier_no_fence();
  int t = 0;
  for (; t + 3 <= n_t; t += 3) {
    step(0, t);
    step(1, t + 1);
    step(2, t + 2);
  }
  if (t < n_t) step(0, t);
  if (t + 1 < n_t) step(1, t + 1);

  // ---- epilogue: lane = key, registers = head_dim 32 db + 8 g4 + 4 hh + 0..3
  if (!k_ok) return;
  float* dvp = p.dv + b * p.dv_sb + h * p.dv_sh + (int64_t)kj * p.dv_ss;
  float* dkp = p.dk + b * p.dk_sb + h * p.dk_sh + (int64_t)kj * p.dk_ss;
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const int d = db * 32 + 8 * g4 + 4 * hh;
      f32x4 v4, k4;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v4[i] = acc_dv[db][4 * g4 + i];
        k4[i] = acc_dk[db][4 * g4 + i] * p.scale;
      }
      *reinterpret_cast<f32x4*>(dvp + d) = v4;
      *reinterpret_cast<f32x4*>(dkp + d) = k4;
    }
}

// ------------------------------------------------------------------------- dQ
__global__ __launch_bounds__(kBwdWaves * 64, 1) void attn_bwd_dq_kernel(BwdParams p) {
  constexpr int LPW = (kTileBytes / 1024) / kBwdWaves;
  constexpr int LOADS = 2 * LPW;
  static_assert(LPW * kBwdWaves * 1024 == kTileBytes, "tile/threads mismatch");

  __shared__ __attribute__((aligned(1024))) unsigned char lk0[kTileBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char lk1[kTileBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char lk2[kTileBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char lv0[kTileBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char lv1[kTileBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char lv2[kTileBytes];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hh = lane >> 5;

  const int n_qblk = (p.Sq + kBwdBlk - 1) / kBwdBlk;
  const int item = xcd_remap(blockIdx.x, gridDim.x);
  const int qblk = item % n_qblk, bh = item / n_qblk;
  const int h = bh % p.H, b = bh / p.H;
  const int qi = qblk * kBwdBlk + wave * 32 + l32;
  const bool q_ok = qi < p.Sq;
  const __bf16* qp = static_cast<const __bf16*>(p.q) + b * p.q_sb + h * p.q_sh;
  const __bf16* kp = static_cast<const __bf16*>(p.k) + b * p.k_sb + h * p.k_sh;
  const __bf16* vp = static_cast<const __bf16*>(p.v) + b * p.v_sb + h * p.v_sh;
  const __bf16* dop = static_cast<const __bf16*>(p.dout) + b * p.do_sb + h * p.do_sh;

  // Q and dO of this lane's query: the B operands of S^T = K Q^T and
  // dP^T = V dO^T. Rows past Sq get LSE = +inf, so their P is 0.
  bf16x8 qf[8], df[8];
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    qf[s] = q_ok ? *reinterpret_cast<const bf16x8*>(qp + (int64_t)qi * p.q_ss + 16 * s + 8 * hh)
                 : bf16x8{};
    df[s] = q_ok ? *reinterpret_cast<const bf16x8*>(dop + (int64_t)qi * p.do_ss + 16 * s + 8 * hh)
                 : bf16x8{};
  }
  float lse2 = __builtin_inff(), delta = 0.0f;
  if (q_ok) {
    const float* a = p.aux + ((int64_t)bh * p.n_qt + qi / kBwdQT) * kAuxRow + (qi % kBwdQT);
    lse2 = a[0];
    delta = a[kBwdQT];
  }

  const uint32_t k_rb = (uint32_t)(p.k_ss * 2), v_rb = (uint32_t)(p.v_ss * 2);
  const int k_rec = (int)((uint32_t)(p.Skv - 1) * k_rb + kD * 2);
  const int v_rec = (int)((uint32_t)(p.Skv - 1) * v_rb + kD * 2);
  uint32_t koff[LPW], voff[LPW];
#pragma unroll
  for (int j = 0; j < LPW; ++j) {
    const int r = 4 * (wave * LPW + j) + (lane >> 4);
    const uint32_t c16 = (uint32_t)swz_v(r, lane & 15) << 4;
    koff[j] = (uint32_t)r * k_rb + c16;
    voff[j] = (uint32_t)r * v_rb + c16;
  }
  const i32x4 k_rsrc = make_rsrc(kp, k_rec), v_rsrc = make_rsrc(vp, v_rec);
  auto kslot = [&](int s) __device__ -> unsigned char* { return s == 0 ? lk0 : s == 1 ? lk1 : lk2; };
  auto vslot = [&](int s) __device__ -> unsigned char* { return s == 0 ? lv0 : s == 1 ? lv1 : lv2; };
  auto issue = [&](int t, int s) __device__ {
    const uint32_t bk = (uint32_t)t * kBN * k_rb, bv = (uint32_t)t * kBN * v_rb;
    const uint32_t dst_k = lds_addr(kslot(s)) + wave * LPW * 1024;
    const uint32_t dst_v = lds_addr(vslot(s)) + wave * LPW * 1024;
#pragma unroll
    for (int j = 0; j < LPW; ++j) lds_dma16(dst_k + j * 1024, koff[j] + bk, k_rsrc);
#pragma unroll
    for (int j = 0; j < LPW; ++j) lds_dma16(dst_v + j * 1024, voff[j] + bv, v_rsrc);
  };

  uint32_t rofs[8];
#pragma unroll
  for (int s = 0; s < 8; ++s) rofs[s] = (uint32_t)(l32 * 256 + (swz_v(l32, 2 * s + hh) << 4));
  uint32_t tofs[2][4];
  tr_offsets(lane, tofs);

  const float c = p.scale_log2;
  f32x16 acc[4];   // dQ^T: [head_dim][query], query = lane
#pragma unroll
  for (int db = 0; db < 4; ++db) acc[db] = f32x16{};

  auto compute = [&](int s, int t) __device__ {
    const unsigned char* tk = kslot(s);
    const LDS_AS unsigned char* lk = (LDS_AS const unsigned char*)tk;
    const LDS_AS unsigned char* lv = (LDS_AS const unsigned char*)vslot(s);
    const int lim = p.Skv - t * kBN - 4 * hh;   // keys at tile offset >= lim + 4 hh are past Skv
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      // S^T and dP^T of keys 32 kb + 8 (r / 4) + 4 hh + r % 4 (register r)
      // and this lane's query
      f32x16 st = f32x16{}, dpt = f32x16{};
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const bf16x8 ak = *(LDS_AS const bf16x8*)(lk + kb * 8192 + rofs[i]);
        const bf16x8 av = *(LDS_AS const bf16x8*)(lv + kb * 8192 + rofs[i]);
        st = mfma16(ak, qf[i], st);
        dpt = mfma16(av, df[i], dpt);
      }
      if (t * kBN + kBN > p.Skv) {
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (32 * kb + 8 * (r >> 2) + (r & 3) >= lim) st[r] = kNegInf;
      }
      bf16x8 pds[2];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float pr = __builtin_amdgcn_exp2f(__builtin_fmaf(st[r], c, -lse2));
        pds[r >> 3][r & 7] = (__bf16)(pr * (dpt[r] - delta));
      }
#pragma unroll
      for (int jj = 0; jj < 2; ++jj)
#pragma unroll
        for (int db = 0; db < 4; ++db)
          acc[db] = mfma16(tr_read(tk, tofs, (kb * 2 + jj) * 4 + db), pds[jj], acc[db]);
    }
  };

  const int n_t = (p.Skv + kBN - 1) / kBN;
  auto step = [&](int s, int t) __device__ {
    if (t + 2 < n_t) issue(t + 2, (s + 2) % 3);
    compute(s, t);
    if (t + 1 < n_t) {
      if (t + 2 < n_t) wait_vmcnt<LOADS>();
      else wait_vmcnt<0>();
      barrier_no_fence();
    }
  };
  issue(0, 0);
  if (n_t > 1) {
    issue(1, 1);
    wait_vmcnt<LOADS>();
  } else {
    wait_vmcnt<0>();
  }
  barrier_no_fence();
  int t = 0;
  for (; t + 3 <= n_t; t += 3) {
    step(0, t);
    step(1, t + 1);
    step(2, t + 2);
  }
  if (t < n_t) step(0, t);
  if (t + 1 < n_t) step(1, t + 1);

  // ---- epilogue: lane = query, registers = head_dim 32 db + 8 g4 + 4 hh + 0..3
  if (!q_ok) return;
  float* dqp = p.dq + b * p.dq_sb + h * p.dq_sh + (int64_t)qi * p.dq_ss;
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const int d = db * 32 + 8 * g4 + 4 * hh;
      f32x4 q4;
#pragma unroll
      for (int i = 0; i < 4; ++i) q4[i] = acc[db][4 * g4 + i] * p.scale;
      *reinterpret_cast<f32x4*>(dqp + d) = q4;
    }
}

}  // namespace

hipError_t launch_attn_bwd(const BwdParams& p, hipStream_t s) {
  const int64_t bh = (int64_t)p.B * p.H;
  const int64_t rows = (int64_t)p.n_qt * kBwdQT;
  hipLaunchKernelGGL(attn_bwd_rows_kernel, dim3((unsigned)(bh * rows / 16)), dim3(256), 0, s, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t n_kblk = (p.Skv + kBwdBlk - 1) / kBwdBlk;
  hipLaunchKernelGGL(attn_bwd_dkdv_kernel, dim3((unsigned)(bh * n_kblk)), dim3(kBwdWaves * 64), 0,
                     s, p);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t n_qblk = (p.Sq + kBwdBlk - 1) / kBwdBlk;
  hipLaunchKernelGGL(attn_bwd_dq_kernel, dim3((unsigned)(bh * n_qblk)), dim3(kBwdWaves * 64), 0, s,
                     p);
  return hipGetLastError();
}

}  // namespace lsh
