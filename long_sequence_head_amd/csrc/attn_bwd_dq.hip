// dQ pass of the attention backward (gfx950); the other passes and the
// definitions are in attn_bwd.hip. Two kernels with the same bits:
// attn_bwd_dq8_kernel (two wavefronts per SIMD, 256 queries per workgroup)
// unless its grid would leave CUs idle where the pipelined
// attn_bwd_dq_kernel's (128 queries per workgroup) would not.
#include "attn_bwd_common.hpp"

namespace lsh {
namespace {

// ------------------------------------------------------------------------- dQ
// Units of 32 keys (two per 64-key tile): A(u) is S^T and dP^T (16 MFMAs,
// queries in lanes), E(u) masks keys past Skv and forms dS^T (bf16, packed
// as the B operand of the next product), B(u) is dQ^T += K^T dS^T (8
// MFMAs). The loop runs A(u+1) interleaved with E(u), then B(u): the
// elementwise work of one unit hides under the matrix work of the next
// (both units' S^T and dP^T are live, which the VGPR budget of this pass
// allows). Tiles, slots and barriers are as in the dK/dV pass.
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
  auto rowread = [&](const unsigned char* tile, int kb, int i) __device__ -> bf16x8 {
    return *(LDS_AS const bf16x8*)((LDS_AS const unsigned char*)tile + kb * 8192 + rofs[i]);
  };

  const float c = p.scale_log2;
  f32x16 acc[4];   // dQ^T: [head_dim][query], query = lane
#pragma unroll
  for (int db = 0; db < 4; ++db) acc[db] = f32x16{};
  f32x16 sA, dA, sB, dB;   // S^T and dP^T of two consecutive units:
                           // register r <-> key 32 kb + 8 (r / 4) + 4 hh + r % 4
  bf16x8 pds[2];

  // keys of the unit starting at key0 that lie past Skv get S = -inf
  auto mask_unit = [&](f32x16& st, int key0) __device__ {
    if (key0 + 32 > p.Skv) {
      const int lim = p.Skv - key0 - 4 * hh;
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (8 * (r >> 2) + (r & 3) >= lim) st[r] = kNegInf;
    }
  };

  auto phase_a = [&](const bool DO_A, const unsigned char* tk, const unsigned char* tv, int ka,
                     const bool DO_E, f32x16& st, f32x16& dpt, const f32x16& se,
                     const f32x16& de) __device__ {
    bf16x8 fk[8], fv[8];
    if (DO_A) {
      fk[0] = rowread(tk, ka, 0);
      fv[0] = rowread(tv, ka, 0);
      fk[1] = rowread(tk, ka, 1);
      fv[1] = rowread(tv, ka, 1);
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if (DO_A) {
        const int k = i >> 1;
        if ((i & 1) == 0) {
          if (k + 2 < 8) fk[k + 2] = rowread(tk, ka, k + 2);
          st = mfma16(fk[k], qf[k], k == 0 ? f32x16{} : st);
        } else {
          if (k + 2 < 8) fv[k + 2] = rowread(tv, ka, k + 2);
          dpt = mfma16(fv[k], df[k], k == 0 ? f32x16{} : dpt);
        }
      }
      if (DO_E) {
        const int r = i;
        const float x = __builtin_amdgcn_exp2f(__builtin_fmaf(se[r], c, -lse2));
        asm volatile("" ::"v"(x));   // computed here, next to this MFMA
        pds[r >> 3][r & 7] = (__bf16)(x * (de[r] - delta));
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  auto phase_b = [&](const unsigned char* tk, int kb) __device__ {
    bf16x8 f[8];
    f[0] = tr_read(tk, tofs, (kb * 2) * 4 + 0);
    f[1] = tr_read(tk, tofs, (kb * 2) * 4 + 1);
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      if (m + 2 < 8) f[m + 2] = tr_read(tk, tofs, (kb * 2 + ((m + 2) >> 2)) * 4 + ((m + 2) & 3));
      acc[m & 3] = mfma16(f[m], pds[m >> 2], acc[m & 3]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  const int n_t = (p.Skv + kBN - 1) / kBN;
  auto step = [&](int s, int t, const bool HAS_NEXT) __device__ {
    const unsigned char* tk = kslot(s);
    const unsigned char* tv = vslot(s);
    const int s1 = (s + 1) % 3;
    mask_unit(sA, t * kBN);
    phase_a(true, tk, tv, 1, true, sB, dB, sA, dA);
    phase_b(tk, 0);
    if (HAS_NEXT) {
      wait_vmcnt<0>();   // tile t+1 (the only loads in flight)
      barrier_no_fence();
      if (t + 2 < n_t) issue(t + 2, (s + 2) % 3);
    }
    mask_unit(sB, t * kBN + 32);
    phase_a(HAS_NEXT, kslot(s1), vslot(s1), 0, true, sA, dA, sB, dB);
    phase_b(tk, 1);
  };

  issue(0, 0);
  if (n_t > 1) {
    issue(1, 1);
    wait_vmcnt<LOADS>();
  } else {
    wait_vmcnt<0>();
  }
  barrier_no_fence();
  phase_a(true, lk0, lv0, 0, false, sA, dA, sA, dA);
  int t = 0;
  for (; t + 3 < n_t; t += 3) {
    step(0, t, true);
    step(1, t + 1, true);
    step(2, t + 2, true);
  }
  const int rest = n_t - t;   // 1, 2 or 3
  if (rest == 3) {
    step(0, t, true);
    step(1, t + 1, true);
    step(2, t + 2, false);
  } else if (rest == 2) {
    step(0, t, true);
    step(1, t + 1, false);
  } else {
    step(0, t, false);
  }

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


// ------------------------------------------- dQ, two wavefronts per SIMD
// Eight wavefronts of 32 queries (256 per workgroup), one workgroup per
// CU, so two wavefronts share each SIMD; each runs the plain order per
// 32-key unit: A (S^T and dP^T, 16 MFMAs), E (dS^T), B (dQ^T += K^T dS^T,
// 8 MFMAs). Every query's operations and their order are those of the
// pipelined kernel above, so both give the same bits. K/V tiles: three
// slots, loaded two ahead, one barrier per tile.
constexpr int kDq8Waves = 8;
constexpr int kDq8Blk = kDq8Waves * 32;
constexpr int kDq8Slots = 3;

__global__ __launch_bounds__(kDq8Waves * 64, 1) void attn_bwd_dq8_kernel(BwdParams p) {
  constexpr int LPW = (kTileBytes / 1024) / kDq8Waves;
  static_assert(LPW * kDq8Waves * 1024 == kTileBytes, "tile/threads mismatch");

  __shared__ __attribute__((aligned(1024))) unsigned char lk[kDq8Slots][kTileBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char lv[kDq8Slots][kTileBytes];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hh = lane >> 5;

  const int n_qblk = (p.Sq + kDq8Blk - 1) / kDq8Blk;
  const int item = xcd_remap(blockIdx.x, gridDim.x);
  const int qblk = item % n_qblk, bh = item / n_qblk;
  const int h = bh % p.H, b = bh / p.H;
  const int qi = qblk * kDq8Blk + wave * 32 + l32;
  const bool q_ok = qi < p.Sq;
  const __bf16* qp = static_cast<const __bf16*>(p.q) + b * p.q_sb + h * p.q_sh;
  const __bf16* kp = static_cast<const __bf16*>(p.k) + b * p.k_sb + h * p.k_sh;
  const __bf16* vp = static_cast<const __bf16*>(p.v) + b * p.v_sb + h * p.v_sh;
  const __bf16* dop = static_cast<const __bf16*>(p.dout) + b * p.do_sb + h * p.do_sh;

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
  // every load above has landed before the first tile load (the compiler
  // does not see those, and would otherwise wait for them in the loop)
  wait_vmcnt<0>();

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
  auto issue = [&](int t, int s) __device__ {
    const uint32_t bk = (uint32_t)t * kBN * k_rb, bv = (uint32_t)t * kBN * v_rb;
    const uint32_t dst_k = lds_addr(lk[s]) + wave * LPW * 1024;
    const uint32_t dst_v = lds_addr(lv[s]) + wave * LPW * 1024;
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
  auto rowread = [&](const unsigned char* tile, int kb, int i) __device__ -> bf16x8 {
    return *(LDS_AS const bf16x8*)((LDS_AS const unsigned char*)tile + kb * 8192 + rofs[i]);
  };

  const float c = p.scale_log2;
  f32x16 acc[4];   // dQ^T: [head_dim][query], query = lane
#pragma unroll
  for (int db = 0; db < 4; ++db) acc[db] = f32x16{};

  const int n_t = (p.Skv + kBN - 1) / kBN;
  // unit kb (keys 32 kb .. 32 kb + 31) of the tile in slot s
  auto unit = [&](int s, int t, int kb) __device__ {
    const unsigned char* tk = lk[s];
    const unsigned char* tv = lv[s];
    f32x16 st, dpt;   // register r <-> key 32 kb + 8 (r / 4) + 4 hh + r % 4
    bf16x8 fk[8], fv[8];
    fk[0] = rowread(tk, kb, 0);
    fv[0] = rowread(tv, kb, 0);
    fk[1] = rowread(tk, kb, 1);
    fv[1] = rowread(tv, kb, 1);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      if (k + 2 < 8) fk[k + 2] = rowread(tk, kb, k + 2);
      st = mfma16(fk[k], qf[k], k == 0 ? f32x16{} : st);
      if (k + 2 < 8) fv[k + 2] = rowread(tv, kb, k + 2);
      dpt = mfma16(fv[k], df[k], k == 0 ? f32x16{} : dpt);
    }
    const int key0 = t * kBN + 32 * kb;
    if (key0 + 32 > p.Skv) {
      const int lim = p.Skv - key0 - 4 * hh;
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (8 * (r >> 2) + (r & 3) >= lim) st[r] = kNegInf;
    }
    bf16x8 pds[2];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float x = __builtin_amdgcn_exp2f(__builtin_fmaf(st[r], c, -lse2));
      pds[r >> 3][r & 7] = (__bf16)(x * (dpt[r] - delta));
    }
    bf16x8 f[8];
    f[0] = tr_read(tk, tofs, (kb * 2) * 4 + 0);
    f[1] = tr_read(tk, tofs, (kb * 2) * 4 + 1);
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      if (m + 2 < 8) f[m + 2] = tr_read(tk, tofs, (kb * 2 + ((m + 2) >> 2)) * 4 + ((m + 2) & 3));
      acc[m & 3] = mfma16(f[m], pds[m >> 2], acc[m & 3]);
    }
  };
  auto advance = [&](int s, int t) __device__ {
    if (t + 1 < n_t) {
      if (t + 2 < n_t) wait_vmcnt<2 * LPW>();   // tile t+2 may stay in flight
      else wait_vmcnt<0>();
      barrier_no_fence();
      if (t + 3 < n_t) issue(t + 3, s);
    }
  };

  issue(0, 0);
  if (n_t > 2) {
    issue(1, 1);
    issue(2, 2);
    wait_vmcnt<4 * LPW>();
  } else if (n_t > 1) {
    issue(1, 1);
    wait_vmcnt<2 * LPW>();
  } else {
    wait_vmcnt<0>();
  }
  barrier_no_fence();
  int t = 0;
  for (; t + kDq8Slots <= n_t; t += kDq8Slots) {
#pragma unroll
    for (int j = 0; j < kDq8Slots; ++j) {
      unit(j, t + j, 0);
      unit(j, t + j, 1);
      advance(j, t + j);
    }
  }
#pragma unroll
  for (int j = 0; j < kDq8Slots - 1; ++j) {
    if (t < n_t) {
      unit(j, t, 0);
      unit(j, t, 1);
      advance(j, t);
      ++t;
    }
  }

  // ---- epilogue (addresses derived again, see the forward kernels)
  int tid2 = (int)threadIdx.x;
  asm volatile("" : "+v"(tid2));
  const int item2 = xcd_remap(blockIdx.x, gridDim.x);
  const int bh2 = item2 / n_qblk;
  const int qi2 = (item2 % n_qblk) * kDq8Blk + (tid2 >> 6) * 32 + (tid2 & 31);
  if (qi2 >= p.Sq) return;
  float* dqp = p.dq + (bh2 / p.H) * p.dq_sb + (bh2 % p.H) * p.dq_sh + (int64_t)qi2 * p.dq_ss;
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

hipError_t launch_attn_bwd_dq(const BwdParams& p, hipStream_t s) {
  const int64_t bh = (int64_t)p.B * p.H;
  const int64_t n8 = bh * ((p.Sq + kDq8Blk - 1) / kDq8Blk);
  if (prefer_two_waves(n8, bh * ((p.Sq + kBwdBlk - 1) / kBwdBlk), p.n_cu)) {
    hipLaunchKernelGGL(attn_bwd_dq8_kernel, dim3((unsigned)n8), dim3(kDq8Waves * 64), 0, s, p);
    return hipGetLastError();
  }
  const int64_t n_qblk = (p.Sq + kBwdBlk - 1) / kBwdBlk;
  hipLaunchKernelGGL(attn_bwd_dq_kernel, dim3((unsigned)(bh * n_qblk)), dim3(kBwdWaves * 64), 0, s,
                     p);
  return hipGetLastError();
}

}  // namespace lsh
