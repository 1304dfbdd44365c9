// C ABI of libpa.so: host-side validation, workspace sizing and dispatch.
//
// Every entry point checks its host arguments before making any HIP call, so
// a rejected call enqueues nothing and needs no GPU.  See include/pa.h for
// the contract of each function.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <algorithm>
#include <atomic>
#include <mutex>

#include "pa.h"
#include "pa_blocks.h"
#include "pa_internal.h"
#include "pa_kernels.h"

namespace pa {

static thread_local char g_last_error[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return code;
}

int ok() {
  g_last_error[0] = '\0';
  return PA_OK;
}

KernelEvents& kernel_events() {
  static thread_local KernelEvents ev{};
  return ev;
}

}  // namespace pa

namespace {

using pa::fail;
using pa::ok;

int hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(PA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// Compute units of the current device, queried once per device.
int device_cus() {
  constexpr int kMaxDevices = 64;
  static std::atomic<int> cache[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  if (dev >= 0 && dev < kMaxDevices) {
    const int c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    n = 256;
  if (dev >= 0 && dev < kMaxDevices) cache[dev].store(n, std::memory_order_relaxed);
  return n;
}

bool supported_head_dim(int d) { return d == 64 || d == 128; }
bool supported_block_size(int b) { return b == 16 || b == 32 || b == 256; }
bool supported_group(int g) { return g == 1 || g == 2 || g == 4 || g == 8; }
bool supported_dtype(int t) { return t == PA_F16 || t == PA_BF16; }
// The softmax scale is a positive temperature (1/sqrt(head_dim) in the pages'
// attention).  The matrix-core kernels take each row's maximum over the raw
// scores and fold the scale into the exponent, which orders scores correctly
// only for a positive scale.
bool valid_scale(float s) { return std::isfinite(s) && s > 0.f; }

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// Scratch of pa_decode_step_scratch, the entry point for callers that cannot
// allocate: the split-K partial results (normalised outputs and fp32 max/sum)
// that pa_decode_step keeps in the caller's workspace.  Every device the
// library runs on holds its own copy until the process ends; each call
// rewrites every byte it later reads, so nothing in it needs clearing.
constexpr size_t kScratchBytes = size_t(16) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

// Device address of a file-scope __device__ variable on the device that runs
// `stream` (the current device for the null stream).  Host code never uses such
// a variable's name as an address: it is looked up with hipGetSymbolAddress
// once per device, with that device current, and kept in `cached`.
constexpr int kMaxDevices = 64;

int device_symbol(hipStream_t stream, const void* symbol, const char* name,
                  void* (&cached)[kMaxDevices], void** addr) {
  static std::mutex mu;
  int dev = -1;
  hipError_t e;
  if (stream) {
    hipDevice_t d = -1;
    e = hipStreamGetDevice(stream, &d);
    dev = (int)d;
  } else {
    e = hipGetDevice(&dev);
  }
  if (e != hipSuccess) return fail(PA_ERR_HIP, "device of the stream: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(PA_ERR_UNSUPPORTED, "device %d: the library serves devices 0..%d", dev,
                kMaxDevices - 1);
  std::lock_guard<std::mutex> lock(mu);
  if (!cached[dev]) {
    int current = -1;
    e = hipGetDevice(&current);
    if (e != hipSuccess) return fail(PA_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
    if (current != dev && (e = hipSetDevice(dev)) != hipSuccess)
      return fail(PA_ERR_HIP, "hipSetDevice(%d): %s", dev, hipGetErrorString(e));
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, symbol);
    if (current != dev) {
      const hipError_t e2 = hipSetDevice(current);
      if (e2 != hipSuccess) return fail(PA_ERR_HIP, "hipSetDevice(%d): %s", current, hipGetErrorString(e2));
    }
    if (e != hipSuccess || !p)
      return fail(PA_ERR_HIP, "hipGetSymbolAddress(%s) on device %d: %s", name, dev,
                  hipGetErrorString(e));
    cached[dev] = p;
  }
  *addr = cached[dev];
  return PA_OK;
}

int scratch_address(hipStream_t stream, void** addr) {
  static void* cached[kMaxDevices] = {};
  return device_symbol(stream, &HIP_SYMBOL(scratch), "scratch", cached, addr);
}

#ifdef PA_CHECK_INDICES
// The index errors the kernels of this (checking) build record, one record
// per device (see IndexErrors); read and cleared by pa_take_index_errors.
static __device__ pa::IndexErrors index_errors;
#endif

// Where this call's kernels record index errors: the device's record in a
// PA_CHECK_INDICES build (after every host check: the first HIP call), null
// otherwise (no HIP call).
int index_errors_address(hipStream_t stream, pa::IndexErrors** addr) {
#ifdef PA_CHECK_INDICES
  static void* cached[kMaxDevices] = {};
  void* p = nullptr;
  const int st = device_symbol(stream, &HIP_SYMBOL(index_errors), "index_errors", cached, &p);
  *addr = static_cast<pa::IndexErrors*>(p);
  return st;
#else
  (void)stream;
  *addr = nullptr;
  return PA_OK;
#endif
}

// Every kernel translation unit's fingerprint of the launch-argument structs
// (pa_kernels.h), compared with this unit's once, when the library is loaded.
const char* layout_error() {
  static char msg[320];
  static const bool bad = [] {
    struct Probe {
      const char* unit;
      uint64_t (*fn)();
    };
    const Probe probes[] = {{"reshape_and_cache.hip", pa::layout_probe_reshape_and_cache},
                            {"rope_reshape.hip", pa::layout_probe_rope_reshape},
                            {"reshape_int8.hip", pa::layout_probe_reshape_int8},
                            {"copy_blocks.hip", pa::layout_probe_copy_blocks},
                            {"decode_f16.hip", pa::layout_probe_decode_f16},
                            {"decode_bf16.hip", pa::layout_probe_decode_bf16},
                            {"decode_int8.hip", pa::layout_probe_decode_int8},
                            {"merge_partials.hip", pa::layout_probe_merge_partials},
                            {"prefill.hip", pa::layout_probe_prefill}};
    const uint64_t mine = pa::args_layout();
    for (const Probe& pr : probes) {
      const uint64_t theirs = pr.fn();
      if (theirs != mine) {
        snprintf(msg, sizeof(msg),
                 "library build mismatch: %s was compiled with another layout of the kernel "
                 "launch arguments (fingerprint %016llx, this unit %016llx); rebuild the whole "
                 "library from one source tree",
                 pr.unit, (unsigned long long)theirs, (unsigned long long)mine);
        return true;
      }
    }
    return false;
  }();
  return bad ? msg : nullptr;
}

[[maybe_unused]] const char* const g_layout_error_at_load = layout_error();

// First check of every entry point that launches kernels.
int check_build() {
  if (const char* m = layout_error()) return fail(PA_ERR_HIP, "%s", m);
  return PA_OK;
}

int64_t num_partitions(int max_context_len, int partition_size) {
  if (partition_size <= 0 || max_context_len <= partition_size) return 1;
  return (max_context_len + (int64_t)partition_size - 1) / partition_size;
}

// Partial outputs first, then the (max, sum) pairs, each 256-byte aligned.
size_t workspace_bytes_for(int num_seqs, int num_heads, int head_dim, int64_t parts) {
  if (parts <= 1) return 0;
  const size_t rows = (size_t)num_seqs * (size_t)num_heads * (size_t)parts;
  return align_up(rows * (size_t)head_dim * sizeof(uint16_t)) + align_up(rows * 2 * sizeof(float));
}

// Shared checks of the paged-cache description.
int check_cache(int num_heads, int num_kv_heads, int head_dim, int block_size, int64_t num_blocks,
                int max_blocks, int dtype) {
  if (num_heads < 1 || num_kv_heads < 1)
    return fail(PA_ERR_INVALID_ARG, "num_heads (%d) and num_kv_heads (%d) must be >= 1", num_heads,
                num_kv_heads);
  if (num_heads % num_kv_heads != 0)
    return fail(PA_ERR_INVALID_ARG, "num_heads (%d) is not a multiple of num_kv_heads (%d)",
                num_heads, num_kv_heads);
  if (!supported_group(num_heads / num_kv_heads))
    return fail(PA_ERR_UNSUPPORTED, "query heads per KV head %d not in {1,2,4,8}",
                num_heads / num_kv_heads);
  if (!supported_head_dim(head_dim))
    return fail(PA_ERR_UNSUPPORTED, "head_dim %d not in {64,128}", head_dim);
  if (!supported_block_size(block_size))
    return fail(PA_ERR_UNSUPPORTED, "block_size %d not in {16,32,256}", block_size);
  if (!supported_dtype(dtype)) return fail(PA_ERR_UNSUPPORTED, "dtype %d not PA_F16/PA_BF16", dtype);
  if (num_blocks < 1) return fail(PA_ERR_INVALID_ARG, "num_blocks must be >= 1");
  if (max_blocks < 1) return fail(PA_ERR_INVALID_ARG, "max_blocks_per_seq must be >= 1");
  if ((int64_t)max_blocks * block_size > INT32_MAX)
    return fail(PA_ERR_INVALID_ARG, "max_blocks_per_seq * block_size exceeds 2^31-1");
  if ((int64_t)num_kv_heads * head_dim * 2 * block_size > (int64_t)1 << 30)
    return fail(PA_ERR_INVALID_ARG, "one cache block exceeds 1 GiB");
  return PA_OK;
}

}  // namespace

extern "C" {

int pa_version(void) { return (1 << 16) | 0; }

const char* pa_status_string(int status) {
  switch (status) {
    case PA_OK: return "PA_OK";
    case PA_ERR_INVALID_ARG: return "PA_ERR_INVALID_ARG: invalid argument";
    case PA_ERR_UNSUPPORTED: return "PA_ERR_UNSUPPORTED: configuration not built";
    case PA_ERR_WORKSPACE: return "PA_ERR_WORKSPACE: workspace missing or too small";
    case PA_ERR_HIP: return "PA_ERR_HIP: HIP runtime error";
    case PA_ERR_NO_BLOCKS: return "PA_ERR_NO_BLOCKS: too few free blocks";
    case PA_ERR_BAD_INDEX: return "PA_ERR_BAD_INDEX: kernels met out-of-range block ids, slots or lengths";
    default: return "unknown pa_status";
  }
}

const char* pa_last_error(void) { return pa::g_last_error; }

int pa_check_indices_enabled(void) {
#ifdef PA_CHECK_INDICES
  return 1;
#else
  return 0;
#endif
}

int pa_take_index_errors(void* stream, uint32_t* kinds, uint32_t* first_kind,
                         int64_t* first_value) {
  if (const int b = check_build()) return b;
  if (!kinds || !first_kind || !first_value) return fail(PA_ERR_INVALID_ARG, "null pointer argument");
  *kinds = 0;
  *first_kind = 0;
  *first_value = 0;
#ifdef PA_CHECK_INDICES
  hipStream_t s = static_cast<hipStream_t>(stream);
  pa::IndexErrors* dev = nullptr;
  if (const int e = index_errors_address(s, &dev)) return e;
  hipError_t e = hipStreamSynchronize(s);
  if (e != hipSuccess) return fail(PA_ERR_HIP, "hipStreamSynchronize: %s", hipGetErrorString(e));
  pa::IndexErrors rec{};
  e = hipMemcpy(&rec, dev, sizeof(rec), hipMemcpyDeviceToHost);
  if (e != hipSuccess) return fail(PA_ERR_HIP, "reading the index-error record: %s", hipGetErrorString(e));
  const pa::IndexErrors zero{};
  e = hipMemcpy(dev, &zero, sizeof(zero), hipMemcpyHostToDevice);
  if (e != hipSuccess) return fail(PA_ERR_HIP, "clearing the index-error record: %s", hipGetErrorString(e));
  *kinds = rec.kinds;
  *first_kind = rec.first_kind;
  *first_value = rec.first_value;
  if (rec.kinds != 0)
    return fail(PA_ERR_BAD_INDEX, "index errors 0x%x; first: kind 0x%x, value %lld", rec.kinds,
                rec.first_kind, (long long)rec.first_value);
  return ok();
#else
  (void)stream;
  return fail(PA_ERR_UNSUPPORTED,
              "this library is built without PA_CHECK_INDICES; index checks are in libpa_check.so");
#endif
}

int pa_set_kernel_events(void* start_event, void* stop_event) {
  if (start_event != nullptr && stop_event == nullptr)
    return fail(PA_ERR_INVALID_ARG, "a start event needs a stop event");
  pa::KernelEvents& ev = pa::kernel_events();
  ev.start = static_cast<hipEvent_t>(start_event);
  ev.stop = static_cast<hipEvent_t>(stop_event);
  ev.start_pending = start_event != nullptr;
  return ok();
}

namespace {
int read_buffer(const void* buf, size_t bytes, bool non_temporal, void* stream) {
  if (bytes == 0) return ok();
  if (buf == nullptr) return fail(PA_ERR_INVALID_ARG, "null buffer");
  if ((reinterpret_cast<uintptr_t>(buf) & 15) != 0 || (bytes & 15) != 0)
    return fail(PA_ERR_INVALID_ARG, "buffer address and size must be multiples of 16 bytes");
  if (const int b = check_build()) return b;
  return hip_status(pa::launch_cache_flush(buf, (int64_t)(bytes / 16), non_temporal,
                                           static_cast<hipStream_t>(stream)),
                    non_temporal ? "stream_read launch" : "cache_flush launch");
}
}  // namespace

int pa_cache_flush(const void* buf, size_t bytes, void* stream) {
  return read_buffer(buf, bytes, false, stream);
}

int pa_stream_read(const void* buf, size_t bytes, void* stream) {
  return read_buffer(buf, bytes, true, stream);
}

int pa_copy_blocks(void* k_cache, void* v_cache, const int64_t* src, const int64_t* dst,
                   int64_t num_copies, int num_kv_heads, int head_dim, int block_size,
                   int64_t num_blocks, int dtype, void* stream) {
  if (const int b = check_build()) return b;
  if (num_copies < 0) return fail(PA_ERR_INVALID_ARG, "num_copies %lld < 0", (long long)num_copies);
  if (!supported_head_dim(head_dim)) return fail(PA_ERR_UNSUPPORTED, "head_dim %d not supported", head_dim);
  if (!supported_block_size(block_size))
    return fail(PA_ERR_UNSUPPORTED, "block_size %d not supported", block_size);
  if (!supported_dtype(dtype)) return fail(PA_ERR_UNSUPPORTED, "dtype %d not supported", dtype);
  if (num_kv_heads <= 0 || num_blocks <= 0)
    return fail(PA_ERR_INVALID_ARG, "num_kv_heads %d / num_blocks %lld must be positive", num_kv_heads,
                (long long)num_blocks);
  if (num_copies == 0) return ok();
  if (!k_cache || !v_cache || !src || !dst) return fail(PA_ERR_INVALID_ARG, "NULL pointer");
  pa::CopyBlocksArgs a;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.src = src;
  a.dst = dst;
  a.num_copies = num_copies;
  a.num_blocks = num_blocks;
  a.block_chunks = (int64_t)block_size * num_kv_heads * head_dim * 2 / 16;
  if (const int e = index_errors_address(static_cast<hipStream_t>(stream), &a.index_errors)) return e;
  return hip_status(pa::launch_copy_blocks(a, static_cast<hipStream_t>(stream)), "copy_blocks launch");
}

int pa_reshape_and_cache(const void* key, const void* value, void* k_cache, void* v_cache,
                         const int64_t* slot_mapping, int64_t num_tokens, int num_kv_heads,
                         int head_dim, int block_size, int64_t num_blocks, int dtype,
                         void* stream) {
  if (const int b = check_build()) return b;
  if (num_tokens < 0) return fail(PA_ERR_INVALID_ARG, "num_tokens must be >= 0");
  if (num_kv_heads < 1) return fail(PA_ERR_INVALID_ARG, "num_kv_heads must be >= 1");
  if (!supported_head_dim(head_dim))
    return fail(PA_ERR_UNSUPPORTED, "head_dim %d not in {64,128}", head_dim);
  if (!supported_block_size(block_size))
    return fail(PA_ERR_UNSUPPORTED, "block_size %d not in {16,32,256}", block_size);
  if (!supported_dtype(dtype)) return fail(PA_ERR_UNSUPPORTED, "dtype %d not PA_F16/PA_BF16", dtype);
  if (num_blocks < 1) return fail(PA_ERR_INVALID_ARG, "num_blocks must be >= 1");
  if (num_tokens == 0) return ok();
  if (!key || !value || !k_cache || !v_cache || !slot_mapping)
    return fail(PA_ERR_INVALID_ARG, "null pointer argument");
  if ((int64_t)num_kv_heads * head_dim * 2 > INT32_MAX / 2)
    return fail(PA_ERR_INVALID_ARG, "token row too large");
  pa::ReshapeArgs a;
  a.key = key;
  a.value = value;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.slot_mapping = slot_mapping;
  a.num_tokens = num_tokens;
  a.num_slots = num_blocks * (int64_t)block_size;
  a.row_chunks = num_kv_heads * head_dim * 2 / 16;
  if (const int e = index_errors_address(static_cast<hipStream_t>(stream), &a.index_errors)) return e;
  return hip_status(pa::launch_reshape_and_cache(a, static_cast<hipStream_t>(stream)),
                    "reshape_and_cache launch");
}

int pa_decode_partition_hint(int num_seqs, int num_kv_heads, int max_context_len,
                             int block_size) {
  if (num_seqs <= 0 || num_kv_heads <= 0 || max_context_len < 0)
    return fail(PA_ERR_INVALID_ARG, "partition hint: non-positive count or negative length");
  if (!supported_block_size(block_size))
    return fail(PA_ERR_UNSUPPORTED, "block_size %d not supported", block_size);
  ok();
  const int64_t slots = 2LL * device_cus();  // decode workgroups resident at once
  const int64_t pairs = (int64_t)num_seqs * num_kv_heads;
  if (pairs >= slots || max_context_len == 0) return 0;
  const int64_t parts = (4 * slots + pairs - 1) / pairs;  // partitions per longest context
  int64_t p = std::max<int64_t>(512, (max_context_len + parts - 1) / parts);
  p = (p + block_size - 1) / block_size * block_size;
  return p >= max_context_len ? 0 : (int)p;
}

size_t pa_decode_workspace_size(int num_seqs, int num_heads, int head_dim, int max_context_len,
                                int partition_size) {
  if (num_seqs <= 0 || num_heads <= 0 || head_dim <= 0 || max_context_len <= 0) return 0;
  return workspace_bytes_for(num_seqs, num_heads, head_dim,
                             num_partitions(max_context_len, partition_size));
}

}  // extern "C"

namespace {

struct NewTokens {
  const void* key;
  const void* value;
  const int64_t* slot_mapping;
  void* k_cache;
  void* v_cache;
  // Rotary embedding of the step (pa_decode_step_rope); null otherwise.
  const int64_t* positions = nullptr;
  const float* cos_table = nullptr;
  const float* sin_table = nullptr;
  int64_t max_position = 0;
  // INT8 caches (pa_decode_step_int8): where the new rows' scales are stored.
  float* k_scales = nullptr;
  float* v_scales = nullptr;
};

// Per-row scales of an INT8 cache (pa_decode_int8); null for 16-bit caches.
struct Int8Scales {
  const float* k;
  const float* v;
};

int decode_impl(void* out, const void* q, const void* k_cache, const void* v_cache,
                const int32_t* block_tables, const int32_t* context_lens,
                const int32_t* seq_order, const NewTokens* nt, const Int8Scales* i8,
                float* out_ml, int num_seqs, int num_heads,
                int num_kv_heads, int head_dim, int block_size, int64_t num_blocks,
                int max_blocks_per_seq, int max_context_len, float scale, int partition_size,
                void* workspace, size_t workspace_bytes, int dtype, void* stream,
                int phases = pa::kPhaseAll, bool use_scratch = false) {
  if (const int b = check_build()) return b;
  if (num_seqs < 0) return fail(PA_ERR_INVALID_ARG, "num_seqs must be >= 0");
  int st = check_cache(num_heads, num_kv_heads, head_dim, block_size, num_blocks,
                       max_blocks_per_seq, dtype);
  if (st != PA_OK) return st;
  if (max_context_len < 0 || (int64_t)max_context_len > (int64_t)max_blocks_per_seq * block_size)
    return fail(PA_ERR_INVALID_ARG, "max_context_len %d outside [0, max_blocks_per_seq*block_size]",
                max_context_len);
  if (!valid_scale(scale)) return fail(PA_ERR_INVALID_ARG, "scale must be finite and > 0");
  if (partition_size < 0 || (partition_size > 0 && partition_size % block_size != 0))
    return fail(PA_ERR_INVALID_ARG, "partition_size %d must be 0 or a positive multiple of %d",
                partition_size, block_size);
  if (num_seqs == 0) return ok();
  if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens)
    return fail(PA_ERR_INVALID_ARG, "null pointer argument");
  if (nt && (!nt->key || !nt->value || !nt->slot_mapping || !nt->k_cache || !nt->v_cache))
    return fail(PA_ERR_INVALID_ARG, "null pointer argument");
  if (nt && i8 && (!nt->k_scales || !nt->v_scales))
    return fail(PA_ERR_INVALID_ARG, "null pointer argument");
  if (i8 && (!i8->k || !i8->v)) return fail(PA_ERR_INVALID_ARG, "null pointer argument");
  if (out_ml && reinterpret_cast<uintptr_t>(out_ml) % 8 != 0)
    return fail(PA_ERR_INVALID_ARG, "out_ml must be 8-byte aligned");
  const int64_t parts = num_partitions(max_context_len, partition_size);
  const int64_t grid = (int64_t)num_seqs * num_kv_heads * parts;
  if (grid > INT32_MAX || (int64_t)num_seqs * num_heads > INT32_MAX)
    return fail(PA_ERR_INVALID_ARG, "launch grid too large");
  const size_t need = workspace_bytes_for(num_seqs, num_heads, head_dim, parts);
  if (need > 0 && use_scratch) {
    if (need > kScratchBytes)
      return fail(PA_ERR_WORKSPACE,
                  "the split needs %zu bytes of workspace; the static scratch holds %zu (use a "
                  "larger partition_size, or pa_decode_step with a workspace)", need, kScratchBytes);
    // Every host check has passed: the scratch address is the first HIP call.
    workspace_bytes = kScratchBytes;
    const int st2 = scratch_address(static_cast<hipStream_t>(stream), &workspace);
    if (st2 != PA_OK) return st2;
  } else if (need > 0) {
    if (!workspace) return fail(PA_ERR_WORKSPACE, "workspace of %zu bytes required", need);
    if (workspace_bytes < need)
      return fail(PA_ERR_WORKSPACE, "workspace has %zu bytes, %zu required", workspace_bytes, need);
    if (reinterpret_cast<uintptr_t>(workspace) % 16 != 0)
      return fail(PA_ERR_WORKSPACE, "workspace must be 16-byte aligned");
  }

  pa::DecodeArgs a;
  a.out = out;
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  const size_t rows = (size_t)num_seqs * num_heads * (size_t)parts;
  a.part_out = need ? static_cast<uint16_t*>(workspace) : nullptr;
  a.part_ml = need ? reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                             align_up(rows * head_dim * sizeof(uint16_t)))
                   : nullptr;
  a.out_ml = out_ml;
  a.seq_order = seq_order;
  a.key_new = nt ? nt->key : nullptr;
  a.value_new = nt ? nt->value : nullptr;
  a.slot_mapping = nt ? nt->slot_mapping : nullptr;
  a.k_cache_w = nt ? nt->k_cache : nullptr;
  a.v_cache_w = nt ? nt->v_cache : nullptr;
  a.k_scales = i8 ? i8->k : nullptr;
  a.v_scales = i8 ? i8->v : nullptr;
  a.k_scales_w = nt ? nt->k_scales : nullptr;
  a.v_scales_w = nt ? nt->v_scales : nullptr;
  a.positions = nt ? nt->positions : nullptr;
  a.rope_cos = nt ? nt->cos_table : nullptr;
  a.rope_sin = nt ? nt->sin_table : nullptr;
  a.max_position = nt ? nt->max_position : 0;
  a.num_slots = num_blocks * (int64_t)block_size;
  a.num_blocks = num_blocks;
  a.num_seqs = num_seqs;
  a.num_heads = num_heads;
  a.num_kv_heads = num_kv_heads;
  a.max_blocks = max_blocks_per_seq;
  a.max_context_len = max_context_len;
  a.num_parts = (int)parts;
  a.part_tokens = parts > 1 ? partition_size : (max_context_len > 0 ? max_context_len : 1);
  a.num_cus = device_cus();
  a.scale_log2 = (float)((double)scale * 1.4426950408889634);  // log2(e)
  const int group = num_heads / num_kv_heads;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (const int e = index_errors_address(s, &a.index_errors)) return e;
  // PA_F16 / PA_BF16 are the kernels' dtype codes.
  hipError_t e = i8 ? pa::launch_decode_int8(a, dtype, head_dim, block_size, group, phases, s)
                 : dtype == PA_BF16 ? pa::launch_decode_bf16(a, head_dim, block_size, group, phases, s)
                                    : pa::launch_decode_f16(a, head_dim, block_size, group, phases, s);
  return hip_status(e, "decode launch");
}

}  // namespace

extern "C" {

int pa_decode(void* out, const void* q, const void* k_cache, const void* v_cache,
              const int32_t* block_tables, const int32_t* context_lens, const int32_t* seq_order,
              int num_seqs, int num_heads, int num_kv_heads, int head_dim, int block_size,
              int64_t num_blocks, int max_blocks_per_seq, int max_context_len, float scale,
              int partition_size, void* workspace, size_t workspace_bytes, int dtype,
              void* stream) {
  return decode_impl(out, q, k_cache, v_cache, block_tables, context_lens, seq_order, nullptr, nullptr, nullptr,
                     num_seqs, num_heads, num_kv_heads, head_dim, block_size, num_blocks,
                     max_blocks_per_seq, max_context_len, scale, partition_size, workspace,
                     workspace_bytes, dtype, stream);
}

int pa_decode_partitions(void* out, const void* q, const void* k_cache, const void* v_cache,
                         const int32_t* block_tables, const int32_t* context_lens,
                         const int32_t* seq_order, int num_seqs, int num_heads, int num_kv_heads,
                         int head_dim, int block_size, int64_t num_blocks, int max_blocks_per_seq,
                         int max_context_len, float scale, int partition_size, void* workspace,
                         size_t workspace_bytes, int dtype, void* stream) {
  return decode_impl(out, q, k_cache, v_cache, block_tables, context_lens, seq_order, nullptr, nullptr,
                     nullptr, num_seqs, num_heads, num_kv_heads, head_dim, block_size, num_blocks,
                     max_blocks_per_seq, max_context_len, scale, partition_size, workspace,
                     workspace_bytes, dtype, stream, pa::kPhasePartitions);
}

int pa_decode_merge(void* out, const int32_t* context_lens, const int32_t* seq_order,
                    int num_seqs, int num_heads, int head_dim, int max_context_len,
                    int partition_size, void* workspace, size_t workspace_bytes, int dtype,
                    void* stream) {
  if (const int b = check_build()) return b;
  if (num_seqs < 0) return fail(PA_ERR_INVALID_ARG, "num_seqs must be >= 0");
  if (num_heads < 1) return fail(PA_ERR_INVALID_ARG, "num_heads must be >= 1");
  if (!supported_head_dim(head_dim))
    return fail(PA_ERR_UNSUPPORTED, "head_dim %d not in {64,128}", head_dim);
  if (!supported_dtype(dtype)) return fail(PA_ERR_UNSUPPORTED, "dtype %d not PA_F16/PA_BF16", dtype);
  if (max_context_len < 0) return fail(PA_ERR_INVALID_ARG, "max_context_len must be >= 0");
  if (partition_size < 0) return fail(PA_ERR_INVALID_ARG, "partition_size must be >= 0");
  const int64_t parts = num_partitions(max_context_len, partition_size);
  if (num_seqs == 0 || parts <= 1) return ok();  // no context spans two partitions
  if (!out || !context_lens) return fail(PA_ERR_INVALID_ARG, "null pointer argument");
  if ((int64_t)num_seqs * num_heads > INT32_MAX) return fail(PA_ERR_INVALID_ARG, "launch grid too large");
  const size_t need = workspace_bytes_for(num_seqs, num_heads, head_dim, parts);
  if (!workspace) return fail(PA_ERR_WORKSPACE, "workspace of %zu bytes required", need);
  if (workspace_bytes < need)
    return fail(PA_ERR_WORKSPACE, "workspace has %zu bytes, %zu required", workspace_bytes, need);
  if (reinterpret_cast<uintptr_t>(workspace) % 16 != 0)
    return fail(PA_ERR_WORKSPACE, "workspace must be 16-byte aligned");
  pa::DecodeArgs a{};
  const size_t rows = (size_t)num_seqs * num_heads * (size_t)parts;
  a.out = out;
  a.context_lens = context_lens;
  a.seq_order = seq_order;
  a.part_out = static_cast<uint16_t*>(workspace);
  a.part_ml = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                       align_up(rows * head_dim * sizeof(uint16_t)));
  a.num_seqs = num_seqs;
  a.num_heads = num_heads;
  a.num_kv_heads = 1;
  a.max_context_len = max_context_len;
  a.num_parts = (int)parts;
  a.part_tokens = partition_size;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (const int e = index_errors_address(s, &a.index_errors)) return e;
  // The merge alone depends on neither the block size nor the head grouping.
  const hipError_t e = dtype == PA_BF16
                           ? pa::launch_decode_bf16(a, head_dim, 16, 1, pa::kPhaseMerge, s)
                           : pa::launch_decode_f16(a, head_dim, 16, 1, pa::kPhaseMerge, s);
  return hip_status(e, "decode merge launch");
}

int pa_decode_step(void* out, const void* q, const void* key, const void* value,
                   const int64_t* slot_mapping, void* k_cache, void* v_cache,
                   const int32_t* block_tables, const int32_t* context_lens,
                   const int32_t* seq_order, int num_seqs, int num_heads, int num_kv_heads,
                   int head_dim, int block_size, int64_t num_blocks, int max_blocks_per_seq,
                   int max_context_len, float scale, int partition_size, void* workspace,
                   size_t workspace_bytes, int dtype, void* stream) {
  NewTokens nt{key, value, slot_mapping, k_cache, v_cache};
  return decode_impl(out, q, k_cache, v_cache, block_tables, context_lens, seq_order, &nt, nullptr, nullptr,
                     num_seqs, num_heads, num_kv_heads, head_dim, block_size, num_blocks,
                     max_blocks_per_seq, max_context_len, scale, partition_size, workspace,
                     workspace_bytes, dtype, stream);
}

int pa_decode_step_scratch(void* out, const void* q, const void* key, const void* value,
                           const int64_t* slot_mapping, void* k_cache, void* v_cache,
                           const int32_t* block_tables, const int32_t* context_lens,
                           const int32_t* seq_order, int num_seqs, int num_heads, int num_kv_heads,
                           int head_dim, int block_size, int64_t num_blocks,
                           int max_blocks_per_seq, int max_context_len, float scale,
                           int partition_size, int dtype, void* stream) {
  NewTokens nt{key, value, slot_mapping, k_cache, v_cache};
  return decode_impl(out, q, k_cache, v_cache, block_tables, context_lens, seq_order, &nt, nullptr,
                     nullptr, num_seqs, num_heads, num_kv_heads, head_dim, block_size, num_blocks,
                     max_blocks_per_seq, max_context_len, scale, partition_size, nullptr, 0, dtype,
                     stream, pa::kPhaseAll, /*use_scratch=*/true);
}

int pa_rope_reshape_and_cache(void* q, const void* key, const void* value, void* k_cache,
                              void* v_cache, const int64_t* positions, const float* cos_table,
                              const float* sin_table, const int64_t* slot_mapping,
                              int64_t num_tokens, int num_heads, int num_kv_heads, int head_dim,
                              int block_size, int64_t num_blocks, int64_t max_position, int dtype,
                              void* stream) {
  if (const int b = check_build()) return b;
  if (num_tokens < 0) return fail(PA_ERR_INVALID_ARG, "num_tokens must be >= 0");
  if (num_kv_heads < 1) return fail(PA_ERR_INVALID_ARG, "num_kv_heads must be >= 1");
  if (q && num_heads < 1) return fail(PA_ERR_INVALID_ARG, "num_heads must be >= 1 with q");
  if (!supported_head_dim(head_dim))
    return fail(PA_ERR_UNSUPPORTED, "head_dim %d not in {64,128}", head_dim);
  if (!supported_block_size(block_size))
    return fail(PA_ERR_UNSUPPORTED, "block_size %d not in {16,32,256}", block_size);
  if (!supported_dtype(dtype)) return fail(PA_ERR_UNSUPPORTED, "dtype %d not PA_F16/PA_BF16", dtype);
  if (num_blocks < 1) return fail(PA_ERR_INVALID_ARG, "num_blocks must be >= 1");
  if (max_position < 1) return fail(PA_ERR_INVALID_ARG, "max_position must be >= 1");
  if (num_tokens == 0) return ok();
  if (!key || !value || !k_cache || !v_cache || !positions || !cos_table || !sin_table ||
      !slot_mapping)
    return fail(PA_ERR_INVALID_ARG, "null pointer argument");
  const void* ptrs[] = {q, key, value, k_cache, v_cache, cos_table, sin_table};
  for (const void* p : ptrs)
    if (reinterpret_cast<uintptr_t>(p) % 16 != 0)
      return fail(PA_ERR_INVALID_ARG, "q, key, value, caches and tables must be 16-byte aligned");
  const int64_t rows = (q ? (int64_t)num_heads : 0) + 2 * (int64_t)num_kv_heads;
  if (rows * head_dim > INT32_MAX / 2) return fail(PA_ERR_INVALID_ARG, "token rows too large");
  pa::RopeReshapeArgs a;
  a.q = q;
  a.key = key;
  a.value = value;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.positions = positions;
  a.cos = cos_table;
  a.sin = sin_table;
  a.slot_mapping = slot_mapping;
  a.num_tokens = num_tokens;
  a.num_slots = num_blocks * (int64_t)block_size;
  a.max_position = max_position;
  a.num_heads = q ? num_heads : 0;
  a.num_kv_heads = num_kv_heads;
  if (const int e = index_errors_address(static_cast<hipStream_t>(stream), &a.index_errors)) return e;
  return hip_status(pa::launch_rope_reshape(a, dtype, head_dim, static_cast<hipStream_t>(stream)),
                    "rope_reshape_and_cache launch");
}

int pa_decode_partial(void* out, float* out_ml, const void* q, const void* k_cache,
                      const void* v_cache, const int32_t* block_tables, const int32_t* context_lens,
                      const int32_t* seq_order, int num_seqs, int num_heads, int num_kv_heads,
                      int head_dim, int block_size, int64_t num_blocks, int max_blocks_per_seq,
                      int max_context_len, float scale, int partition_size, void* workspace,
                      size_t workspace_bytes, int dtype, void* stream) {
  if (num_seqs > 0 && !out_ml) return fail(PA_ERR_INVALID_ARG, "null pointer argument");
  return decode_impl(out, q, k_cache, v_cache, block_tables, context_lens, seq_order, nullptr, nullptr,
                     out_ml, num_seqs, num_heads, num_kv_heads, head_dim, block_size, num_blocks,
                     max_blocks_per_seq, max_context_len, scale, partition_size, workspace,
                     workspace_bytes, dtype, stream);
}

int pa_merge_partials(void* out, float* out_ml, const void* partial_o, const float* partial_ml,
                      int num_shards, int num_seqs, int num_heads, int head_dim, int dtype,
                      void* stream) {
  if (const int b = check_build()) return b;
  if (num_shards < 1) return fail(PA_ERR_INVALID_ARG, "num_shards must be >= 1");
  if (num_seqs < 0) return fail(PA_ERR_INVALID_ARG, "num_seqs must be >= 0");
  if (num_heads < 1) return fail(PA_ERR_INVALID_ARG, "num_heads must be >= 1");
  if (!supported_head_dim(head_dim))
    return fail(PA_ERR_UNSUPPORTED, "head_dim %d not in {64,128}", head_dim);
  if (!supported_dtype(dtype)) return fail(PA_ERR_UNSUPPORTED, "dtype %d not PA_F16/PA_BF16", dtype);
  const int64_t rows = (int64_t)num_seqs * num_heads;
  if (rows > INT32_MAX) return fail(PA_ERR_INVALID_ARG, "launch grid too large");
  if (rows == 0) return ok();
  if (!out || !partial_o || !partial_ml) return fail(PA_ERR_INVALID_ARG, "null pointer argument");
  if (reinterpret_cast<uintptr_t>(partial_ml) % 8 != 0 ||
      (out_ml && reinterpret_cast<uintptr_t>(out_ml) % 8 != 0))
    return fail(PA_ERR_INVALID_ARG, "partial_ml and out_ml must be 8-byte aligned");
  if (reinterpret_cast<uintptr_t>(partial_o) % 4 != 0)
    return fail(PA_ERR_INVALID_ARG, "partial_o must be 4-byte aligned");
  pa::MergePartialsArgs a;
  a.out = out;
  a.out_ml = out_ml;
  a.part_o = partial_o;
  a.part_ml = partial_ml;
  a.num_rows = rows;
  a.num_shards = num_shards;
  return hip_status(pa::launch_merge_partials(a, dtype, head_dim, static_cast<hipStream_t>(stream)),
                    "merge_partials launch");
}

int pa_decode_step_rope(void* out, const void* q, const void* key, const void* value,
                        const int64_t* slot_mapping, const int64_t* positions, const float* cos_table,
                        const float* sin_table, int64_t max_position, void* k_cache, void* v_cache,
                        const int32_t* block_tables, const int32_t* context_lens,
                        const int32_t* seq_order, int num_seqs, int num_heads, int num_kv_heads,
                        int head_dim, int block_size, int64_t num_blocks, int max_blocks_per_seq,
                        int max_context_len, float scale, int partition_size, void* workspace,
                        size_t workspace_bytes, int dtype, void* stream) {
  if (num_seqs > 0) {
    if (!positions || !cos_table || !sin_table)
      return fail(PA_ERR_INVALID_ARG, "null pointer argument");
    if (max_position < 1) return fail(PA_ERR_INVALID_ARG, "max_position must be >= 1");
    if (reinterpret_cast<uintptr_t>(cos_table) % 16 != 0 ||
        reinterpret_cast<uintptr_t>(sin_table) % 16 != 0)
      return fail(PA_ERR_INVALID_ARG, "cos/sin tables must be 16-byte aligned");
  }
  NewTokens nt{key, value, slot_mapping, k_cache, v_cache, positions, cos_table, sin_table,
               max_position};
  return decode_impl(out, q, k_cache, v_cache, block_tables, context_lens, seq_order, &nt, nullptr,
                     nullptr, num_seqs, num_heads, num_kv_heads, head_dim, block_size, num_blocks,
                     max_blocks_per_seq, max_context_len, scale, partition_size, workspace,
                     workspace_bytes, dtype, stream);
}

int pa_reshape_and_cache_int8(const void* key, const void* value, void* k_codes, void* v_codes,
                              float* k_scales, float* v_scales, const int64_t* slot_mapping,
                              int64_t num_tokens, int num_kv_heads, int head_dim, int block_size,
                              int64_t num_blocks, int dtype, void* stream) {
  if (const int b = check_build()) return b;
  if (num_tokens < 0) return fail(PA_ERR_INVALID_ARG, "num_tokens must be >= 0");
  if (num_kv_heads < 1) return fail(PA_ERR_INVALID_ARG, "num_kv_heads must be >= 1");
  if (!supported_head_dim(head_dim))
    return fail(PA_ERR_UNSUPPORTED, "head_dim %d not in {64,128}", head_dim);
  if (!supported_block_size(block_size))
    return fail(PA_ERR_UNSUPPORTED, "block_size %d not in {16,32,256}", block_size);
  if (!supported_dtype(dtype)) return fail(PA_ERR_UNSUPPORTED, "dtype %d not PA_F16/PA_BF16", dtype);
  if (num_blocks < 1) return fail(PA_ERR_INVALID_ARG, "num_blocks must be >= 1");
  if (num_tokens == 0) return ok();
  if (!key || !value || !k_codes || !v_codes || !k_scales || !v_scales || !slot_mapping)
    return fail(PA_ERR_INVALID_ARG, "null pointer argument");
  if ((int64_t)num_kv_heads * head_dim > INT32_MAX / 4)
    return fail(PA_ERR_INVALID_ARG, "token row too large");
  pa::ReshapeInt8Args a;
  a.key = key;
  a.value = value;
  a.k_codes = k_codes;
  a.v_codes = v_codes;
  a.k_scales = k_scales;
  a.v_scales = v_scales;
  a.slot_mapping = slot_mapping;
  a.num_tokens = num_tokens;
  a.num_slots = num_blocks * (int64_t)block_size;
  a.num_kv_heads = num_kv_heads;
  a.block_size = block_size;
  if (const int e = index_errors_address(static_cast<hipStream_t>(stream), &a.index_errors)) return e;
  return hip_status(pa::launch_reshape_int8(a, dtype, head_dim, static_cast<hipStream_t>(stream)),
                    "reshape_and_cache_int8 launch");
}

int pa_decode_int8(void* out, const void* q, const void* k_codes, const void* v_codes,
                   const float* k_scales, const float* v_scales, const int32_t* block_tables,
                   const int32_t* context_lens, const int32_t* seq_order, int num_seqs,
                   int num_heads, int num_kv_heads, int head_dim, int block_size, int64_t num_blocks,
                   int max_blocks_per_seq, int max_context_len, float scale, int partition_size,
                   void* workspace, size_t workspace_bytes, int dtype, void* stream) {
  const Int8Scales i8{k_scales, v_scales};
  return decode_impl(out, q, k_codes, v_codes, block_tables, context_lens, seq_order, nullptr, &i8, nullptr,
                     num_seqs, num_heads, num_kv_heads, head_dim, block_size, num_blocks,
                     max_blocks_per_seq, max_context_len, scale, partition_size, workspace,
                     workspace_bytes, dtype, stream);
}

int pa_decode_step_int8(void* out, const void* q, const void* key, const void* value,
                        const int64_t* slot_mapping, void* k_codes, void* v_codes, float* k_scales,
                        float* v_scales, const int32_t* block_tables, const int32_t* context_lens,
                        const int32_t* seq_order, int num_seqs, int num_heads, int num_kv_heads,
                        int head_dim, int block_size, int64_t num_blocks, int max_blocks_per_seq,
                        int max_context_len, float scale, int partition_size, void* workspace,
                        size_t workspace_bytes, int dtype, void* stream) {
  NewTokens nt{key, value, slot_mapping, k_codes, v_codes};
  nt.k_scales = k_scales;
  nt.v_scales = v_scales;
  const Int8Scales i8{k_scales, v_scales};
  return decode_impl(out, q, k_codes, v_codes, block_tables, context_lens, seq_order, &nt, &i8, nullptr,
                     num_seqs, num_heads, num_kv_heads, head_dim, block_size, num_blocks,
                     max_blocks_per_seq, max_context_len, scale, partition_size, workspace,
                     workspace_bytes, dtype, stream);
}

int pa_decode_order(const int32_t* context_lens, int num_seqs, int32_t* order) {
  if (num_seqs < 0) return fail(PA_ERR_INVALID_ARG, "num_seqs must be >= 0");
  if (num_seqs == 0) return ok();
  if (!context_lens || !order) return fail(PA_ERR_INVALID_ARG, "null pointer argument");
  for (int i = 0; i < num_seqs; ++i) order[i] = i;
  // Longest context first; equal lengths keep their index order.
  std::stable_sort(order, order + num_seqs, [context_lens](int32_t x, int32_t y) {
    return context_lens[x] > context_lens[y];
  });
  return ok();
}

int pa_prefill_chunk(void* out, const void* q, const void* k_cache, const void* v_cache,
                     const int32_t* block_tables, const int32_t* context_lens,
                     const int32_t* query_start_loc, const int32_t* seq_order, int num_seqs,
                     int64_t num_tokens,
                     int num_heads, int num_kv_heads, int head_dim, int block_size,
                     int64_t num_blocks, int max_blocks_per_seq, int max_query_len, float scale,
                     int dtype, void* stream) {
  if (const int b = check_build()) return b;
  if (num_seqs < 0 || num_tokens < 0)
    return fail(PA_ERR_INVALID_ARG, "num_seqs and num_tokens must be >= 0");
  int st = check_cache(num_heads, num_kv_heads, head_dim, block_size, num_blocks,
                       max_blocks_per_seq, dtype);
  if (st != PA_OK) return st;
  if (max_query_len < 0) return fail(PA_ERR_INVALID_ARG, "max_query_len must be >= 0");
  if (!valid_scale(scale)) return fail(PA_ERR_INVALID_ARG, "scale must be finite and > 0");
  if (num_seqs == 0 || num_tokens == 0 || max_query_len == 0) return ok();
  if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens || !query_start_loc)
    return fail(PA_ERR_INVALID_ARG, "null pointer argument");
  if (num_tokens > INT32_MAX) return fail(PA_ERR_INVALID_ARG, "num_tokens exceeds 2^31-1");

  pa::PrefillArgs a;
  a.out = out;
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.query_start_loc = query_start_loc;
  a.seq_order = seq_order;
  a.num_blocks = num_blocks;
  a.num_tokens = num_tokens;
  a.num_seqs = num_seqs;
  a.num_heads = num_heads;
  a.num_kv_heads = num_kv_heads;
  a.max_blocks = max_blocks_per_seq;
  a.max_query_len = max_query_len;
  a.q_tiles = 0;  // chosen by the launcher
  a.scale_log2 = (float)((double)scale * 1.4426950408889634);
  if (const int e = index_errors_address(static_cast<hipStream_t>(stream), &a.index_errors)) return e;
  return hip_status(pa::launch_prefill(a, dtype, head_dim, block_size, num_heads / num_kv_heads,
                                       static_cast<hipStream_t>(stream)),
                    "prefill launch");
}

}  // extern "C"
