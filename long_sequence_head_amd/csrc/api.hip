// C ABI of liblsh.so: argument validation, launch set-up and the
// two-stream head-chunk pipeline. Kernels live in attn_fwd.hip,
// attn_bwd.hip and aux_kernels.hip.
#include "lsh.h"
#include "lsh_internal.hpp"

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

namespace {

thread_local char g_err[512] = "";

lsh_status fail(lsh_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

lsh_status ok() {
  g_err[0] = '\0';
  return LSH_OK;
}

int elem_bytes(int32_t dtype) { return dtype == LSH_F32 ? 4 : 2; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Size and span checks multiply caller-given 64-bit values (sizes below
// 2^30, strides of any value); they are formed in 128 bits so that no
// product wraps.
using wide_t = __int128;
inline wide_t W(int64_t x) { return static_cast<wide_t>(x); }
// a * b * c >= limit for factors >= 1 of any size (limit below 2^31)
inline bool prod3_ge(int64_t a, int64_t b, int64_t c, int64_t limit) {
  if (a >= limit || b >= limit || c >= limit) return true;
  return W(a) * b * c >= limit;
}

constexpr int kMaxDevices = 64;
std::mutex g_dev_mu;
int g_dev_state[kMaxDevices];  // 0 unknown, 1 gfx950, 2 other
int g_dev_cus[kMaxDevices];    // compute units of each checked device
// compute units of the device the calling thread's last successful device
// check found (the kernels' grid-size choices use it)
thread_local int g_cur_cus = 0;

lsh_status device_check_impl() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
    (void)hipGetLastError();
    return fail(LSH_ERR_NO_DEVICE, "no HIP device is available");
  }
  if (dev >= kMaxDevices) return fail(LSH_ERR_NO_DEVICE, "device index %d out of range", dev);
  std::lock_guard<std::mutex> lk(g_dev_mu);
  if (g_dev_state[dev] == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
      (void)hipGetLastError();
      return fail(LSH_ERR_NO_DEVICE, "cannot query device %d", dev);
    }
    g_dev_state[dev] = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
    g_dev_cus[dev] = prop.multiProcessorCount;
  }
  if (g_dev_state[dev] != 1) return fail(LSH_ERR_NO_DEVICE, "device %d is not gfx950", dev);
  g_cur_cus = g_dev_cus[dev];
  return LSH_OK;
}

// Validates an attention argument block. Returns LSH_OK or an error with
// g_err set. No HIP call is made.
lsh_status validate_attn(const lsh_attn_args* a, bool allow_empty_kv, const char* fn) {
  if (!a) return fail(LSH_ERR_INVALID, "%s: args is NULL", fn);
  if (a->dtype != LSH_F32 && a->dtype != LSH_BF16)
    return fail(LSH_ERR_INVALID, "%s: unknown dtype %d", fn, a->dtype);
  if (a->reserved != 0) return fail(LSH_ERR_INVALID, "%s: reserved field must be 0", fn);
  if (a->B < 1 || a->Sq < 1 || a->H < 1 || a->D < 1)
    return fail(LSH_ERR_INVALID, "%s: B, Sq, H, D must be >= 1 (got %lld, %lld, %lld, %lld)", fn,
                (long long)a->B, (long long)a->Sq, (long long)a->H, (long long)a->D);
  if (a->Skv < (allow_empty_kv ? 0 : 1))
    return fail(LSH_ERR_INVALID, "%s: Skv must be >= %d (got %lld)", fn, allow_empty_kv ? 0 : 1,
                (long long)a->Skv);
  if (a->D != LSH_HEAD_DIM)
    return fail(LSH_ERR_UNSUPPORTED, "%s: head_dim %lld is not supported (only %d)", fn,
                (long long)a->D, LSH_HEAD_DIM);
  const int64_t lim = (int64_t)1 << 30;
  if (a->B >= lim || a->Sq >= lim || a->Skv >= lim || a->H >= lim)
    return fail(LSH_ERR_UNSUPPORTED, "%s: sizes must be below 2^30", fn);
  const int64_t qblocks = (a->Sq + 127) / 128;
  const wide_t big = W(1) << 31;
  if (W(a->B) * a->H * qblocks >= big || W(a->B) * a->Sq * a->H >= big)
    return fail(LSH_ERR_UNSUPPORTED, "%s: B*Sq*H too large", fn);
  if (!a->q || !a->o || !a->lse) return fail(LSH_ERR_INVALID, "%s: q, o and lse must be non-NULL", fn);
  const bool need_kv = a->Skv > 0;
  if (need_kv && (!a->k || !a->v)) return fail(LSH_ERR_INVALID, "%s: k and v must be non-NULL", fn);
  if (!std::isfinite(a->scale)) return fail(LSH_ERR_INVALID, "%s: scale must be finite", fn);
  const int eb = elem_bytes(a->dtype);
  const void* ptrs[5] = {a->q, a->k, a->v, a->o, a->lse};
  for (int i = 0; i < 5; ++i)
    if (ptrs[i] && !aligned16(ptrs[i]))
      return fail(LSH_ERR_INVALID, "%s: pointer %d is not 16-byte aligned", fn, i);
  // bf16 K and V rows are read through buffer descriptors with 32-bit byte
  // offsets: one head's rows must span less than 2 GiB.
  if (a->dtype == LSH_BF16 && need_kv) {
    const wide_t span_k = W(a->Skv - 1) * a->k_stride[1] * eb + W(a->D) * eb;
    const wide_t span_v = W(a->Skv - 1) * a->v_stride[1] * eb + W(a->D) * eb;
    if (span_k >= big || span_v >= big)
      return fail(LSH_ERR_UNSUPPORTED,
                  "%s: the K/V rows of one head span 2 GiB or more (Skv x key stride)", fn);
  }
  const int64_t* strides[4] = {a->q_stride, a->k_stride, a->v_stride, a->o_stride};
  const int ebs[4] = {eb, eb, eb, 4};
  for (int t = 0; t < 4; ++t) {
    if (t >= 1 && t <= 2 && !need_kv) continue;
    for (int i = 0; i < 3; ++i) {
      const int64_t st = strides[t][i];
      if (st < 0) return fail(LSH_ERR_INVALID, "%s: negative stride", fn);
      if ((st * ebs[t]) % 16 != 0)
        return fail(LSH_ERR_INVALID, "%s: stride %lld x %d bytes is not a multiple of 16", fn,
                    (long long)st, ebs[t]);
    }
  }
  return LSH_OK;
}

lsh::AttnParams make_params(const lsh_attn_args* a) {
  lsh::AttnParams p;
  std::memset(&p, 0, sizeof(p));
  p.q = a->q;
  p.k = a->k;
  p.v = a->v;
  p.o = a->o;
  p.lse = a->lse;
  p.q_sb = a->q_stride[0];
  p.q_ss = a->q_stride[1];
  p.q_sh = a->q_stride[2];
  p.k_sb = a->k_stride[0];
  p.k_ss = a->k_stride[1];
  p.k_sh = a->k_stride[2];
  p.v_sb = a->v_stride[0];
  p.v_ss = a->v_stride[1];
  p.v_sh = a->v_stride[2];
  p.o_sb = a->o_stride[0];
  p.o_ss = a->o_stride[1];
  p.o_sh = a->o_stride[2];
  p.lse_sb = a->H * a->Sq;
  p.lse_sh = a->Sq;
  p.B = (int32_t)a->B;
  p.H = (int32_t)a->H;
  p.Sq = (int32_t)a->Sq;
  p.Skv = (int32_t)a->Skv;
  p.scale = a->scale;
  p.scale_log2 = (float)((double)a->scale * 1.4426950408889634);  // scale * log2(e)
  p.n_cu = g_cur_cus;
  return p;
}

// Validates a backward argument block (no HIP call).
lsh_status validate_bwd(const lsh_attn_bwd_args* a, const char* fn) {
  if (!a) return fail(LSH_ERR_INVALID, "%s: args is NULL", fn);
  if (a->dtype != LSH_F32 && a->dtype != LSH_BF16)
    return fail(LSH_ERR_INVALID, "%s: unknown dtype %d", fn, a->dtype);
  if (a->reserved != 0) return fail(LSH_ERR_INVALID, "%s: reserved field must be 0", fn);
  if (a->B < 1 || a->Sq < 1 || a->Skv < 1 || a->H < 1 || a->D < 1)
    return fail(LSH_ERR_INVALID, "%s: B, Sq, Skv, H, D must be >= 1", fn);
  if (a->D != LSH_HEAD_DIM)
    return fail(LSH_ERR_UNSUPPORTED, "%s: head_dim %lld is not supported (only %d)", fn,
                (long long)a->D, LSH_HEAD_DIM);
  if (a->dtype != LSH_BF16)
    return fail(LSH_ERR_UNSUPPORTED, "%s: only bf16 inputs are supported", fn);
  const int64_t lim = (int64_t)1 << 30;
  if (a->B >= lim || a->Sq >= lim || a->Skv >= lim || a->H >= lim)
    return fail(LSH_ERR_UNSUPPORTED, "%s: sizes must be below 2^30", fn);
  const wide_t big = W(1) << 31;
  const wide_t bh = W(a->B) * a->H;
  if (bh * ((a->Sq + 127) / 128) >= big || bh * ((a->Skv + 127) / 128) >= big ||
      bh * ((a->Sq + lsh::kBwdQT - 1) / lsh::kBwdQT) * (lsh::kBwdQT / 16) >= big ||
      bh * a->Sq >= big || bh * a->Skv >= big)
    return fail(LSH_ERR_UNSUPPORTED, "%s: B*S*H too large", fn);
  const void* ptrs[9] = {a->q, a->k, a->v, a->dout, a->o, a->lse, a->dq, a->dk, a->dv};
  static const char* names[9] = {"q", "k", "v", "dout", "o", "lse", "dq", "dk", "dv"};
  for (int i = 0; i < 9; ++i) {
    if (!ptrs[i]) return fail(LSH_ERR_INVALID, "%s: %s is NULL", fn, names[i]);
    if (!aligned16(ptrs[i]))
      return fail(LSH_ERR_INVALID, "%s: %s is not 16-byte aligned", fn, names[i]);
  }
  if (!std::isfinite(a->scale)) return fail(LSH_ERR_INVALID, "%s: scale must be finite", fn);
  const int64_t* strides[8] = {a->q_stride, a->k_stride, a->v_stride, a->do_stride,
                               a->o_stride, a->dq_stride, a->dk_stride, a->dv_stride};
  const int ebs[8] = {2, 2, 2, 2, 4, 4, 4, 4};
  for (int t = 0; t < 8; ++t)
    for (int i = 0; i < 3; ++i) {
      const int64_t st = strides[t][i];
      if (st < 0) return fail(LSH_ERR_INVALID, "%s: negative stride", fn);
      if ((st * ebs[t]) % 16 != 0)
        return fail(LSH_ERR_INVALID, "%s: stride %lld x %d bytes is not a multiple of 16", fn,
                    (long long)st, ebs[t]);
    }
  // Q, dO, K and V rows are read through buffer descriptors with 32-bit
  // byte offsets: one head's rows of each must span less than 2 GiB.
  const int64_t rows[4] = {a->Sq, a->Skv, a->Skv, a->Sq};
  for (int t = 0; t < 4; ++t)
    if (W(rows[t] - 1) * strides[t][1] * 2 + W(a->D) * 2 >= big)
      return fail(LSH_ERR_UNSUPPORTED, "%s: the rows of one head span 2 GiB or more", fn);
  return LSH_OK;
}

lsh::BwdParams make_bwd_params(const lsh_attn_bwd_args* a, void* workspace) {
  lsh::BwdParams p;
  std::memset(&p, 0, sizeof(p));
  p.q = a->q;
  p.k = a->k;
  p.v = a->v;
  p.dout = a->dout;
  p.o = a->o;
  p.lse = a->lse;
  p.dq = a->dq;
  p.dk = a->dk;
  p.dv = a->dv;
  p.aux = static_cast<float*>(workspace);
  const int64_t* src[8] = {a->q_stride, a->k_stride, a->v_stride, a->do_stride,
                           a->o_stride, a->dq_stride, a->dk_stride, a->dv_stride};
  int64_t* dst[8][3] = {{&p.q_sb, &p.q_ss, &p.q_sh},    {&p.k_sb, &p.k_ss, &p.k_sh},
                        {&p.v_sb, &p.v_ss, &p.v_sh},    {&p.do_sb, &p.do_ss, &p.do_sh},
                        {&p.o_sb, &p.o_ss, &p.o_sh},    {&p.dq_sb, &p.dq_ss, &p.dq_sh},
                        {&p.dk_sb, &p.dk_ss, &p.dk_sh}, {&p.dv_sb, &p.dv_ss, &p.dv_sh}};
  for (int t = 0; t < 8; ++t)
    for (int i = 0; i < 3; ++i) *dst[t][i] = src[t][i];
  p.lse_sb = a->H * a->Sq;
  p.lse_sh = a->Sq;
  p.B = (int32_t)a->B;
  p.H = (int32_t)a->H;
  p.Sq = (int32_t)a->Sq;
  p.Skv = (int32_t)a->Skv;
  p.scale = a->scale;
  p.scale_log2 = (float)((double)a->scale * 1.4426950408889634);  // scale * log2(e)
  p.n_qt = (int32_t)((a->Sq + lsh::kBwdQT - 1) / lsh::kBwdQT);
  p.n_cu = g_cur_cus;
  return p;
}

lsh_status hip_status(hipError_t e, const char* fn) {
  if (e == hipSuccess) return ok();
  return fail(LSH_ERR_HIP, "%s: %s", fn, hipGetErrorString(e));
}

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Checks of a block-sparse call shared by both entry points (no HIP call).
lsh_status validate_blocksparse(const lsh_attn_args* args, const uint8_t* block_mask,
                                const char* fn) {
  lsh_status st = validate_attn(args, false, fn);
  if (st != LSH_OK) return st;
  if (!block_mask) return fail(LSH_ERR_INVALID, "%s: block_mask is NULL", fn);
  const int64_t n_mkb = (args->Skv + LSH_MASK_BLOCK - 1) / LSH_MASK_BLOCK;
  if (n_mkb > 32768) return fail(LSH_ERR_UNSUPPORTED, "%s: Skv above 2^22 is not supported", fn);
  return LSH_OK;
}

// Enqueues the schedule kernels and the block-sparse kernel (arguments checked).
lsh_status blocksparse_launch(const lsh_attn_args* args, const uint8_t* block_mask,
                              void* workspace, hipStream_t s, const char* fn) {
  const int64_t n_mqb = (args->Sq + LSH_MASK_BLOCK - 1) / LSH_MASK_BLOCK;
  const int64_t n_mkb = (args->Skv + LSH_MASK_BLOCK - 1) / LSH_MASK_BLOCK;
  lsh::AttnParams p = make_params(args);
  p.mask = block_mask;
  p.n_mqb = (int32_t)n_mqb;
  p.n_mkb = (int32_t)n_mkb;
  const int32_t n_items = (int32_t)(args->B * args->H * n_mqb);
  // workspace: int32 counts[n_items] | int32 order[n_items] |
  // int64 totals[B * H] | uint16 kept[n_items][n_mkb] | int32 place[B * H + 8]
  const size_t region = round_up((size_t)n_items * sizeof(int32_t), 256);
  const size_t tot_region = round_up((size_t)(args->B * args->H) * sizeof(long long), 256);
  const size_t kept_region = round_up((size_t)n_items * (size_t)n_mkb * sizeof(unsigned short), 256);
  char* ws = static_cast<char*>(workspace);
  int32_t* counts = reinterpret_cast<int32_t*>(ws);
  int32_t* order = reinterpret_cast<int32_t*>(ws + region);
  long long* totals = reinterpret_cast<long long*>(ws + 2 * region);
  unsigned short* kept = reinterpret_cast<unsigned short*>(ws + 2 * region + tot_region);
  int32_t* place = reinterpret_cast<int32_t*>(ws + 2 * region + tot_region + kept_region);
  hipError_t e = lsh::launch_sparse_schedule(block_mask, n_items, p.n_mkb, p.n_mqb, counts, totals,
                                             order, kept, place, s);
  if (e != hipSuccess) return hip_status(e, fn);
  p.order = order;
  p.counts = counts;
  p.kept = kept;
  return hip_status(lsh::launch_attn_sparse(p, static_cast<lsh::DType>(args->dtype), s), fn);
}


// Static scratch of the allocation-free block-sparse entry point: the
// launch schedule lives here instead of in a caller workspace. Each device
// holds its own copy for the life of the process. In host code `scratch`
// only names the symbol; its device address comes from hipGetSymbolAddress,
// taken once per device with that device current.
constexpr size_t kScratchBytes = LSH_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

// Device address of `scratch` on the current device (checked by the caller).
lsh_status scratch_ptr(void** out, const char* fn) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return fail(LSH_ERR_NO_DEVICE, "%s: no current device", fn);
  }
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      (void)hipGetLastError();
      return fail(LSH_ERR_HIP, "%s: hipGetSymbolAddress(scratch): %s", fn, hipGetErrorString(e));
    }
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return LSH_OK;
}

// Events of the chunk pipeline, created once per device and reused under a
// lock (a stream wait captures the event state at the time of the call).
constexpr int kMaxChunks = 64;
struct EventPool {
  std::mutex mu;
  bool ready = false;
  hipEvent_t ev[kMaxChunks + 1];
};
EventPool g_pools[kMaxDevices];

}  // namespace

extern "C" {

int lsh_abi_version(void) { return LSH_ABI_VERSION; }

const char* lsh_status_str(int status) {
  switch (status) {
    case LSH_OK: return "ok";
    case LSH_ERR_INVALID: return "invalid argument";
    case LSH_ERR_UNSUPPORTED: return "unsupported argument";
    case LSH_ERR_WORKSPACE: return "workspace missing or too small";
    case LSH_ERR_NO_DEVICE: return "no gfx950 device";
    case LSH_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char* lsh_last_error(void) { return g_err; }

lsh_status lsh_device_check(void) {
  lsh_status st = device_check_impl();
  return st == LSH_OK ? ok() : st;
}

lsh_status lsh_attn_fwd(const lsh_attn_args* args, lsh_stream stream) {
  lsh_status st = validate_attn(args, false, "lsh_attn_fwd");
  if (st != LSH_OK) return st;
  if ((st = device_check_impl()) != LSH_OK) return st;
  const lsh::AttnParams p = make_params(args);
  return hip_status(lsh::launch_attn_dense(p, static_cast<lsh::DType>(args->dtype),
                                           static_cast<hipStream_t>(stream)),
                    "lsh_attn_fwd");
}

lsh_status lsh_attn_partial(const lsh_attn_args* args, lsh_stream stream) {
  lsh_status st = validate_attn(args, true, "lsh_attn_partial");
  if (st != LSH_OK) return st;
  if ((st = device_check_impl()) != LSH_OK) return st;
  const lsh::AttnParams p = make_params(args);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (args->Skv == 0) return hip_status(lsh::launch_attn_empty(p, s), "lsh_attn_partial");
  return hip_status(lsh::launch_attn_dense(p, static_cast<lsh::DType>(args->dtype), s),
                    "lsh_attn_partial");
}

lsh_status lsh_attn_partial_accumulate(const lsh_attn_args* args, lsh_stream stream) {
  const char* fn = "lsh_attn_partial_accumulate";
  lsh_status st = validate_attn(args, true, fn);
  if (st != LSH_OK) return st;
  if ((st = device_check_impl()) != LSH_OK) return st;
  if (args->Skv == 0) return ok();   // an empty block leaves the running result as it is
  lsh::AttnParams p = make_params(args);
  p.accumulate = 1;
  return hip_status(lsh::launch_attn_dense(p, static_cast<lsh::DType>(args->dtype),
                                           static_cast<hipStream_t>(stream)),
                    fn);
}

size_t lsh_attn_fwd_chunked_workspace(const lsh_attn_args* args) {
  if (validate_attn(args, false, "lsh_attn_fwd_chunked_workspace") != LSH_OK) return 0;
  const size_t one = (size_t)args->B * args->H * args->Sq * args->D * elem_bytes(args->dtype);
  return 3 * round_up(one, 256);
}

lsh_status lsh_attn_fwd_chunked(const lsh_attn_args* args, const int32_t* head_chunks,
                                int32_t n_chunks, void* workspace, size_t workspace_bytes,
                                lsh_stream compute_stream, lsh_stream permute_stream) {
  const char* fn = "lsh_attn_fwd_chunked";
  lsh_status st = validate_attn(args, false, fn);
  if (st != LSH_OK) return st;
  if (args->Sq != args->Skv) return fail(LSH_ERR_INVALID, "%s: requires Sq == Skv", fn);
  if (!head_chunks) return fail(LSH_ERR_INVALID, "%s: head_chunks is NULL", fn);
  if (n_chunks < 1 || n_chunks > kMaxChunks)
    return fail(LSH_ERR_INVALID, "%s: n_chunks must be in [1, %d]", fn, kMaxChunks);
  int64_t sum = 0;
  for (int i = 0; i < n_chunks; ++i) {
    if (head_chunks[i] < 1) return fail(LSH_ERR_INVALID, "%s: chunk %d is < 1", fn, i);
    sum += head_chunks[i];
  }
  if (sum != args->H)
    return fail(LSH_ERR_INVALID, "%s: chunks sum to %lld, H is %lld", fn, (long long)sum,
                (long long)args->H);
  const size_t need = lsh_attn_fwd_chunked_workspace(args);
  if (!workspace || workspace_bytes < need)
    return fail(LSH_ERR_WORKSPACE, "%s: workspace of %zu bytes needed", fn, need);
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
    return fail(LSH_ERR_WORKSPACE, "%s: workspace must be 256-byte aligned", fn);
  // the permute reads contiguous [B, S, H, D] inputs
  const int64_t HD = args->H * args->D;
  const int64_t* qs[3] = {args->q_stride, args->k_stride, args->v_stride};
  for (int t = 0; t < 3; ++t)
    if (qs[t][0] != args->Sq * HD || qs[t][1] != HD || qs[t][2] != args->D)
      return fail(LSH_ERR_INVALID, "%s: q, k, v must be contiguous [B, S, H, D]", fn);
  if ((st = device_check_impl()) != LSH_OK) return st;

  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return hip_status(hipGetLastError(), fn);
  hipStream_t sc = static_cast<hipStream_t>(compute_stream);
  hipStream_t sp = static_cast<hipStream_t>(permute_stream);
  const bool two = sc != sp;
  const int eb = elem_bytes(args->dtype);
  const size_t one = round_up((size_t)args->B * args->H * args->Sq * args->D * eb, 256);
  char* ws = static_cast<char*>(workspace);
  const void* src[3] = {args->q, args->k, args->v};
  char* dstbase[3] = {ws, ws + one, ws + 2 * one};
  const lsh::DType dt = static_cast<lsh::DType>(args->dtype);

  EventPool& pool = g_pools[dev];
  std::lock_guard<std::mutex> lk(pool.mu);
  if (two && !pool.ready) {
    for (int i = 0; i <= kMaxChunks; ++i)
      if (hipEventCreateWithFlags(&pool.ev[i], hipEventDisableTiming) != hipSuccess)
        return hip_status(hipGetLastError(), fn);
    pool.ready = true;
  }
  hipError_t e;
  if (two) {
    // the permute stream starts after everything already on the compute stream
    if ((e = hipEventRecord(pool.ev[0], sc)) != hipSuccess) return hip_status(e, fn);
    if ((e = hipStreamWaitEvent(sp, pool.ev[0], 0)) != hipSuccess) return hip_status(e, fn);
  }
  int32_t h0 = 0;
  for (int c = 0; c < n_chunks; ++c) {
    const int32_t hc = head_chunks[c];
    const size_t chunk_off = (size_t)args->B * h0 * args->Sq * args->D * eb;
    for (int t = 0; t < 3; ++t) {
      e = lsh::launch_head_permute(src[t], dstbase[t] + chunk_off, eb, args->B, args->Sq, args->H,
                                   args->D, h0, hc, sp);
      if (e != hipSuccess) return hip_status(e, fn);
    }
    if (two) {
      if ((e = hipEventRecord(pool.ev[c + 1], sp)) != hipSuccess) return hip_status(e, fn);
      if ((e = hipStreamWaitEvent(sc, pool.ev[c + 1], 0)) != hipSuccess) return hip_status(e, fn);
    }
    // attention over the chunk's head-major copy: [B, hc, S, D]
    lsh::AttnParams p = make_params(args);
    const int64_t sd = args->Sq * args->D;
    p.q = dstbase[0] + chunk_off;
    p.k = dstbase[1] + chunk_off;
    p.v = dstbase[2] + chunk_off;
    p.q_sb = p.k_sb = p.v_sb = hc * sd;
    p.q_ss = p.k_ss = p.v_ss = args->D;
    p.q_sh = p.k_sh = p.v_sh = sd;
    p.o = args->o + h0 * args->o_stride[2];
    p.lse = args->lse + (int64_t)h0 * args->Sq;
    p.lse_sb = args->H * args->Sq;
    p.lse_sh = args->Sq;
    p.H = hc;
    if ((e = lsh::launch_attn_dense(p, dt, sc)) != hipSuccess) return hip_status(e, fn);
    h0 += hc;
  }
  return ok();
}

lsh_status lsh_lse_merge(const float* o_parts, const float* lse_parts, int32_t n, int64_t B,
                         int64_t Sq, int64_t H, int64_t D, float* o, float* lse,
                         lsh_stream stream) {
  const char* fn = "lsh_lse_merge";
  if (!o_parts || !lse_parts || !o || !lse) return fail(LSH_ERR_INVALID, "%s: NULL pointer", fn);
  if (n < 1 || n > 4096) return fail(LSH_ERR_INVALID, "%s: n must be in [1, 4096]", fn);
  if (B < 1 || Sq < 1 || H < 1 || D < 1) return fail(LSH_ERR_INVALID, "%s: sizes must be >= 1", fn);
  if (D != LSH_HEAD_DIM)
    return fail(LSH_ERR_UNSUPPORTED, "%s: head_dim %lld is not supported", fn, (long long)D);
  if (prod3_ge(B, Sq, H, (int64_t)1 << 31))
    return fail(LSH_ERR_UNSUPPORTED, "%s: too many rows", fn);
  if (!aligned16(o_parts) || !aligned16(o) || !aligned16(lse_parts) || !aligned16(lse))
    return fail(LSH_ERR_INVALID, "%s: pointers must be 16-byte aligned", fn);
  lsh_status st = device_check_impl();
  if (st != LSH_OK) return st;
  return hip_status(lsh::launch_lse_merge(o_parts, lse_parts, n, B, Sq, H, o, lse,
                                          static_cast<hipStream_t>(stream)),
                    fn);
}

lsh_status lsh_head_permute(const void* src, void* dst, int32_t dtype, int64_t B, int64_t S,
                            int64_t H, int64_t D, int32_t h0, int32_t hc, lsh_stream stream) {
  const char* fn = "lsh_head_permute";
  if (!src || !dst) return fail(LSH_ERR_INVALID, "%s: NULL pointer", fn);
  if (dtype != LSH_F32 && dtype != LSH_BF16) return fail(LSH_ERR_INVALID, "%s: unknown dtype", fn);
  if (B < 1 || S < 1 || H < 1 || D < 1) return fail(LSH_ERR_INVALID, "%s: sizes must be >= 1", fn);
  if (h0 < 0 || hc < 1 || (int64_t)h0 + hc > H)
    return fail(LSH_ERR_INVALID, "%s: head range [%d, %d) outside [0, %lld)", fn, h0, h0 + hc,
                (long long)H);
  const int eb = elem_bytes(dtype);
  if ((W(D) * eb) % 16 != 0)
    return fail(LSH_ERR_INVALID, "%s: D * element size must be a multiple of 16", fn);
  if (W(S) * (W(D) * eb / 16) >= (W(1) << 31) || W(B) * hc > 65535)
    return fail(LSH_ERR_UNSUPPORTED, "%s: shape too large", fn);
  if (!aligned16(src) || !aligned16(dst)) return fail(LSH_ERR_INVALID, "%s: pointers must be 16-byte aligned", fn);
  lsh_status st = device_check_impl();
  if (st != LSH_OK) return st;
  return hip_status(lsh::launch_head_permute(src, dst, eb, B, S, H, D, h0, hc,
                                             static_cast<hipStream_t>(stream)),
                    fn);
}

size_t lsh_attn_fwd_blocksparse_workspace(const lsh_attn_args* args) {
  if (validate_attn(args, false, "lsh_attn_fwd_blocksparse_workspace") != LSH_OK) return 0;
  const int64_t n_items = args->B * args->H * ((args->Sq + LSH_MASK_BLOCK - 1) / LSH_MASK_BLOCK);
  const int64_t n_mkb = (args->Skv + LSH_MASK_BLOCK - 1) / LSH_MASK_BLOCK;
  return 2 * round_up((size_t)n_items * sizeof(int32_t), 256) +
         round_up((size_t)(args->B * args->H) * sizeof(long long), 256) +
         round_up((size_t)n_items * (size_t)n_mkb * sizeof(unsigned short), 256) +
         round_up((size_t)(args->B * args->H + 8) * sizeof(int32_t), 256);
}

lsh_status lsh_attn_fwd_blocksparse(const lsh_attn_args* args, const uint8_t* block_mask,
                                    void* workspace, size_t workspace_bytes, lsh_stream stream) {
  const char* fn = "lsh_attn_fwd_blocksparse";
  lsh_status st = validate_blocksparse(args, block_mask, fn);
  if (st != LSH_OK) return st;
  const size_t need = lsh_attn_fwd_blocksparse_workspace(args);
  if (!workspace || workspace_bytes < need)
    return fail(LSH_ERR_WORKSPACE, "%s: workspace of %zu bytes needed", fn, need);
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
    return fail(LSH_ERR_WORKSPACE, "%s: workspace must be 256-byte aligned", fn);
  if ((st = device_check_impl()) != LSH_OK) return st;
  return blocksparse_launch(args, block_mask, workspace, static_cast<hipStream_t>(stream), fn);
}

lsh_status lsh_attn_fwd_blocksparse_noalloc(const lsh_attn_args* args, const uint8_t* block_mask,
                                            lsh_stream stream) {
  const char* fn = "lsh_attn_fwd_blocksparse_noalloc";
  lsh_status st = validate_blocksparse(args, block_mask, fn);
  if (st != LSH_OK) return st;
  const size_t need = lsh_attn_fwd_blocksparse_workspace(args);
  if (need > kScratchBytes)
    return fail(LSH_ERR_WORKSPACE,
                "%s: the schedule needs %zu bytes, more than the %zu-byte static scratch; use "
                "lsh_attn_fwd_blocksparse with a caller workspace",
                fn, need, kScratchBytes);
  if ((st = device_check_impl()) != LSH_OK) return st;
  void* ws = nullptr;
  if ((st = scratch_ptr(&ws, fn)) != LSH_OK) return st;
  return blocksparse_launch(args, block_mask, ws, static_cast<hipStream_t>(stream), fn);
}



size_t lsh_attn_bwd_workspace(const lsh_attn_bwd_args* args) {
  if (validate_bwd(args, "lsh_attn_bwd_workspace") != LSH_OK) return 0;
  const int64_t n_qt = (args->Sq + lsh::kBwdQT - 1) / lsh::kBwdQT;
  return (size_t)(args->B * args->H * n_qt) * (size_t)(2 * lsh::kBwdQT * sizeof(float));
}

lsh_status lsh_attn_bwd(const lsh_attn_bwd_args* args, void* workspace, size_t workspace_bytes,
                        lsh_stream stream) {
  const char* fn = "lsh_attn_bwd";
  lsh_status st = validate_bwd(args, fn);
  if (st != LSH_OK) return st;
  const size_t need = lsh_attn_bwd_workspace(args);
  if (!workspace || workspace_bytes < need)
    return fail(LSH_ERR_WORKSPACE, "%s: workspace of %zu bytes needed", fn, need);
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
    return fail(LSH_ERR_WORKSPACE, "%s: workspace must be 256-byte aligned", fn);
  if ((st = device_check_impl()) != LSH_OK) return st;
  const lsh::BwdParams p = make_bwd_params(args, workspace);
  return hip_status(lsh::launch_attn_bwd(p, static_cast<hipStream_t>(stream)), fn);
}

}  // extern "C"
