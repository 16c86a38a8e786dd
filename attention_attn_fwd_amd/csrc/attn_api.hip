// C ABI of libattn_fwd.so (declared in include/attn_fwd.h): argument checks,
// launch planning, per-stream scratch for the split-KV path, launches.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <climits>
#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <memory>
#include <mutex>
#include <vector>

#include "../../include/attn_fwd.h"
#include "attn_internal.h"

// Scratch of attn_fwd_noalloc (the split-KV partial states): device memory
// that exists on every GPU the library runs on for the life of the process.
// In host code this name is only a stand-in for the symbol; the device
// address is looked up once per device (noalloc_scratch below) and only that
// address is ever passed to a kernel.
constexpr int64_t kNoAllocScratchBytes = (int64_t)64 << 20;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace attn {
namespace {

constexpr int kMaxDevices = 64;

// Scratch of the allocating entry points: one device buffer per (device,
// stream) the library has been called on, grown when a call needs more and
// kept for the next call; calls on different streams get different buffers.
// Each buffer carries an event recorded after the kernels of the last call
// that used it, and a call first makes its stream wait for that event: on
// the same stream the wait is already implied by stream order, and when a
// destroyed stream's handle comes back as a new stream, the new stream's
// call cannot start before the old stream's last call has finished with the
// buffer.  Growing waits on the host for that event, then frees and
// reallocates: rare, and the only host synchronisation these calls make.
// (A stream-ordered pool allocation and free per call made every call wait
// on the host for the stream's earlier work, so no call could be queued
// ahead of the GPU.)  One mutex covers a call from the lookup to the event
// record, so a buffer cannot be regrown while another host thread's call
// that uses it is being enqueued.  Under graph capture the buffer is used as
// it stands (no event operations, which a capture cannot take across its
// boundary); a capture that would need a larger buffer fails.
struct StreamScratch {
  int dev;
  hipStream_t stream;
  void* ptr;
  size_t bytes;
  hipEvent_t last_use;  // null until the first call records it
};
std::mutex g_ws_mutex;
std::vector<std::unique_ptr<StreamScratch>> g_ws;

// Holds the scratch mutex for one call from acquire() on; after the
// launches, record() marks the buffer's last use on the call's stream.
class ScratchCall {
 public:
  ScratchCall() : lock_(g_ws_mutex, std::defer_lock) {}
  // The stream's buffer of at least `bytes` bytes, with `stream` ordered
  // after the buffer's last use.
  int acquire(hipStream_t stream, size_t bytes, void** out);
  int record();

 private:
  std::unique_lock<std::mutex> lock_;
  StreamScratch* slot_ = nullptr;
  hipStream_t stream_ = nullptr;
  bool capturing_ = false;
};

int ScratchCall::acquire(hipStream_t stream, size_t bytes, void** out) {
  const char* fail = std::getenv("ATTN_FWD_FAIL_ALLOC");
  if (fail && fail[0] == '1') return ATTN_ERR_OOM;
  lock_.lock();
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return ATTN_ERR_HIP;
  hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(stream, &cap) != hipSuccess) return ATTN_ERR_HIP;
  capturing_ = cap != hipStreamCaptureStatusNone;
  StreamScratch* e = nullptr;
  for (auto& s : g_ws)
    if (s->dev == dev && s->stream == stream) e = s.get();
  if (!e || e->bytes < bytes) {
    if (capturing_) return ATTN_ERR_HIP;  // a capture can neither wait on the host nor allocate here
    size_t want = bytes;
    if (e) {
      want = std::max(want, e->bytes + e->bytes / 2);
      if (e->last_use && hipEventSynchronize(e->last_use) != hipSuccess) return ATTN_ERR_HIP;
      if (hipFree(e->ptr) != hipSuccess) return ATTN_ERR_HIP;
      e->ptr = nullptr;
      e->bytes = 0;
    } else {
      g_ws.push_back(std::make_unique<StreamScratch>(StreamScratch{dev, stream, nullptr, 0, nullptr}));
      e = g_ws.back().get();
    }
    constexpr size_t kGrain = (size_t)2 << 20;
    want = (want + kGrain - 1) / kGrain * kGrain;
    void* ptr = nullptr;
    if (hipMalloc(&ptr, want) != hipSuccess || !ptr) {
      (void)hipGetLastError();
      return ATTN_ERR_OOM;
    }
    e->ptr = ptr;
    e->bytes = want;
  }
  if (!capturing_ && e->last_use && hipStreamWaitEvent(stream, e->last_use, 0) != hipSuccess) return ATTN_ERR_HIP;
  slot_ = e;
  stream_ = stream;
  *out = e->ptr;
  return ATTN_OK;
}

int ScratchCall::record() {
  if (!slot_ || capturing_) return ATTN_OK;
  if (!slot_->last_use && hipEventCreateWithFlags(&slot_->last_use, hipEventDisableTiming) != hipSuccess) {
    slot_->last_use = nullptr;
    return ATTN_ERR_HIP;
  }
  return hipEventRecord(slot_->last_use, stream_) == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

int release_stream_scratch() {
  std::lock_guard<std::mutex> lock(g_ws_mutex);
  int cur = 0;
  if (hipGetDevice(&cur) != hipSuccess) return ATTN_ERR_HIP;
  int status = ATTN_OK;
  for (auto& s : g_ws) {
    if (hipSetDevice(s->dev) != hipSuccess) {
      status = ATTN_ERR_HIP;
      continue;
    }
    if (s->last_use && hipEventSynchronize(s->last_use) != hipSuccess) status = ATTN_ERR_HIP;
    if (s->ptr && hipFree(s->ptr) != hipSuccess) status = ATTN_ERR_HIP;
    if (s->last_use && hipEventDestroy(s->last_use) != hipSuccess) status = ATTN_ERR_HIP;
  }
  g_ws.clear();
  if (hipSetDevice(cur) != hipSuccess) status = ATTN_ERR_HIP;
  return status;
}

// Device address of `scratch` on each device, looked up on the first
// attn_fwd_noalloc call on that device, with that device current.
struct ScratchSlot {
  std::once_flag once;
  void* ptr = nullptr;
  hipError_t err = hipSuccess;
};
ScratchSlot g_scratch[kMaxDevices];

hipError_t noalloc_scratch(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  ScratchSlot& ss = g_scratch[dev];
  std::call_once(ss.once, [&]() {
    ss.err = hipGetSymbolAddress(&ss.ptr, HIP_SYMBOL(scratch));
    if (ss.err == hipSuccess && !ss.ptr) ss.err = hipErrorInvalidSymbol;
  });
  *out = ss.ptr;
  return ss.err;
}

// Chip geometry, queried once per device: compute units and XCDs (the
// partition mode decides both; a single-XCD partition has no XCD mapping).
// ATTN_FWD_CUS / ATTN_FWD_XCDS override them (tests plan for other chips on
// hosts without a GPU); with no device the MI355X figures stand in.
struct Geometry {
  int cus = 256;
  int xcds = 8;
};
struct GeometrySlot {
  std::once_flag once;
  Geometry g;
};
GeometrySlot g_geometry[kMaxDevices];

Geometry device_geometry() {
  Geometry g;
  int dev = -1;
  if (hipGetDevice(&dev) == hipSuccess && dev >= 0 && dev < kMaxDevices) {
    GeometrySlot& gs = g_geometry[dev];
    std::call_once(gs.once, [&]() {
      int v = 0;
      if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0) gs.g.cus = v;
      v = 0;
      if (hipDeviceGetAttribute(&v, hipDeviceAttributeNumberOfXccs, dev) == hipSuccess && v > 0) gs.g.xcds = v;
      (void)hipGetLastError();
    });
    g = gs.g;
  } else {
    (void)hipGetLastError();
  }
  if (const char* e = std::getenv("ATTN_FWD_CUS")) {
    const int v = std::atoi(e);
    if (v >= 1) g.cus = v;
  }
  if (const char* e = std::getenv("ATTN_FWD_XCDS")) {
    const int v = std::atoi(e);
    if (v >= 1) g.xcds = v;
  }
  return g;
}

// A failed launch is reported through the status code; the runtime's
// per-thread error state it set is consumed so it does not surface later in
// the caller's unrelated HIP calls.
int launch_status(hipError_t e) {
  if (e == hipSuccess) return ATTN_OK;
  (void)hipGetLastError();
  return ATTN_ERR_HIP;
}

// Head widths: multiples of 16 up to 512 on the 16-bit MFMA kernels (above
// 128 the 8-wave prefill forms), up to 128 on the fp32 kernel.
bool supported_width(int d, bool mfma) { return d >= 16 && d <= (mfma ? 512 : 128) && d % 16 == 0; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Workers of the split-KV pass: as many single-wave workgroups as are
// resident at once (four per CU, fewer when the two LDS ring stages of K, V
// and Q sub-blocks of the kernel that launches need more than 40 KiB),
// fewer still when even the padded length gives less than kDecodeMinShare
// sub-blocks each.  ATTN_FWD_SPLIT_WORKERS (>= 1) overrides it.
int split_workers(int B, int Hkv, int K, int D, int Dv, int rows, const Geometry& geo) {
  if (K <= 0) return 0;
  if (const char* e = std::getenv("ATTN_FWD_SPLIT_WORKERS")) {
    const int v = std::atoi(e);
    if (v >= 1) return v;
  }
  int dp = pad_width(D), dvp = pad_width(Dv);
  if (dp > 128 || dvp > 128) dp = dvp = 256;  // the wide decode kernel pads both widths to 256
  const int qrows = rows <= 16 ? 16 : 32;
  const int stage = kDecodeSub * (dp + dvp) * 2 + qrows * dp * 2;
  const int per_cu = std::min(4, 160 * 1024 / (2 * stage));
  const int64_t resident = (int64_t)per_cu * geo.cus;
  const int64_t sub = (int64_t)B * Hkv * ((K + kDecodeSub - 1) / kDecodeSub);
  const int64_t w = (sub + kDecodeMinShare - 1) / kDecodeMinShare;
  return (int)std::max<int64_t>(1, std::min(w, resident));
}

// Key-range pieces per prefill tile.  The kernel holds two workgroups per CU
// (512 on MI355X's 256 CUs); while the tiles alone fill fewer than that, each
// tile's range is cut so that tiles x pieces reaches about that many, keeping
// at least kPrefillMinSplitBlocks 64-key blocks per piece so the partial
// states (the fp32 accumulator of 128 rows, written and read back once: about
// an eighth of the K/V bytes such a piece streams at D = Dv = 128) and the
// combine launch stay small next to the piece.  If that leaves some CUs
// without a workgroup, pieces down to kPrefillMinSplitBlocksIdle blocks are
// taken to give every CU one.  (Measured on MI355X: with 256 workgroups already
// running, 16-block pieces lost to 32-block ones; with 16 running, 16-block
// pieces won; 8-block pieces never paid for the combine launch.)
// ATTN_FWD_PREFILL_SPLITS (>= 1) overrides it.
int prefill_splits(int B, int Hkv, int Q, int group, int K, const Geometry& geo) {
  if (K <= 0) return 1;
  if (const char* e = std::getenv("ATTN_FWD_PREFILL_SPLITS")) {
    const int v = std::atoi(e);
    if (v >= 1) return std::min(v, kPrefillMaxSplits);
  }
  // The combine pass runs one wave per output row, four to a workgroup.
  if ((int64_t)B * Hkv * group * Q > INT32_MAX) return 1;
  const int64_t tiles = (int64_t)B * Hkv * prefill_group_tiles(Q, group);
  const int64_t kSlots = 2 * (int64_t)geo.cus, kCUs = geo.cus;
  const int64_t blocks = ((int64_t)K + kPrefillBN - 1) / kPrefillBN;
  int64_t s = 1;
  if (tiles < kSlots) {
    s = std::min((kSlots + tiles - 1) / tiles, blocks / kPrefillMinSplitBlocks);
    if (tiles * s < kCUs) s = std::max(s, std::min((kCUs + tiles - 1) / tiles, blocks / kPrefillMinSplitBlocksIdle));
  }
  // Lean tiles (at most 64 rows, as in decode with wide heads): their partial
  // states are small next to a piece's K/V, and with lengths that vary one
  // long sequence would otherwise hold a single workgroup for its whole range.
  const int64_t rows = std::min<int64_t>(kPrefillBM, prefill_packed(Q, group) ? (int64_t)group * Q : Q);
  if (rows <= 64) s = std::max(s, blocks / kPrefillMinSplitBlocks);
  return (int)std::max<int64_t>(1, std::min<int64_t>(s, kPrefillMaxSplits));
}

// Blocks per piece when the longest key range (K) is cut into `splits`.
int prefill_split_blocks(int K, int splits) {
  const int blocks = (K + kPrefillBN - 1) / kPrefillBN;
  return (blocks + splits - 1) / splits;
}

// Checks shared by both entry points; fills the plan.
int check_and_plan(int B, int Hq, int Hkv, int Q, int K, int D, int Dv, int window, float scale, bool bf16,
                   const Geometry& geo, attn_fwd_plan_t* plan) {
  (void)window;
  *plan = attn_fwd_plan_t{0, 0, 0, 0};
  if (B < 0 || Hq < 0 || Hkv < 0 || Q < 0 || K < 0 || D < 0 || Dv < 0) return ATTN_ERR_INVALID_ARG;
  if (Hq > 0 && (Hkv == 0 || Hq % Hkv != 0)) return ATTN_ERR_INVALID_ARG;
  if (!std::isfinite(scale)) return ATTN_ERR_INVALID_ARG;
  if ((int64_t)B * Hq * Q == 0) return ATTN_OK;
  if (!supported_width(D, bf16) || !supported_width(Dv, bf16)) return ATTN_ERR_UNSUPPORTED;
  // Byte offsets inside one (batch, head) slice are 32-bit in the kernels, and
  // the buffer loads read a padding channel as zero by giving it an offset
  // of 2^31, past the end of any slice below that size.
  const int64_t lim = (int64_t)1 << 31;
  if ((int64_t)Q * D * 2 >= lim || (int64_t)Q * Dv * 2 >= lim || (int64_t)K * D * 2 >= lim ||
      (int64_t)K * Dv * 2 >= lim)
    return ATTN_ERR_UNSUPPORTED;
  const int group = Hq / Hkv;
  const bool narrow = D <= 128 && Dv <= 128, wide = !narrow && D <= 256 && Dv <= 256;
  if (bf16 && Q <= kDecodeMaxQ && ((narrow && group * Q <= kDecodeMaxRows) || (wide && group * Q <= kDecodeMaxRowsWide))) {
    plan->path = 2;
    plan->split_workers = split_workers(B, Hkv, K, D, Dv, group * Q, geo);
    plan->partial_slots = plan->split_workers > 0 ? B * Hkv + plan->split_workers : 0;
    const int64_t parts = (int64_t)plan->partial_slots * group * Q;
    plan->workspace_bytes = parts * (int64_t)(Dv + 2) * 4;
  } else {
    plan->path = 1;
    const int bm = bf16 ? kPrefillBM : kF32Rows;
    // Workgroup indices are int: tiles x pieces x output-channel parts.
    if ((int64_t)((Q + bm - 1) / bm) * Hq * B > (int64_t)INT32_MAX) return ATTN_ERR_UNSUPPORTED;
    if (bf16) {
      const int64_t tiles = (int64_t)B * Hkv * prefill_group_tiles(Q, group);
      const int dv_parts = (D > 256 || Dv > 256) ? (Dv + 255) / 256 : 1;
      if (tiles * dv_parts > (int64_t)INT32_MAX) return ATTN_ERR_UNSUPPORTED;
      // Pieces of a fixed number of blocks: the requested count rounded to
      // what whole pieces of ceil(blocks / count) blocks need.
      const int want = prefill_splits(B, Hkv, Q, group, K, geo);
      const int blocks = (K + kPrefillBN - 1) / kPrefillBN;
      int ns = want > 1 ? (blocks + prefill_split_blocks(K, want) - 1) / prefill_split_blocks(K, want) : 1;
      if (tiles * ns * dv_parts > (int64_t)INT32_MAX) ns = 1;
      plan->split_workers = ns;
      if (ns > 1) {
        plan->partial_slots = (int)(tiles * ns);
        plan->workspace_bytes = (int64_t)plan->partial_slots * kPrefillBM * (Dv + 2) * 4;
      }
    }
  }
  return ATTN_OK;
}

// A paged K/V cache (null: contiguous k, v).
struct PagedArgs {
  const int32_t* block_table;
  int pages_per_seq, page_shift, num_pages;
};

// flags: ATTN_FWD_FP16 / ATTN_FWD_FP32 select the element type (bf16 when
// neither), ATTN_FWD_NONCAUSAL drops the causal limit.  noalloc: the split-KV
// scratch is the library's static `scratch` (no allocation; a plan that
// needs more returns ATTN_ERR_SCRATCH_LIMIT before anything is launched).
int run(int flags, const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq, int Hkv, int Q,
        int K, int D, int Dv, const int32_t* seqlens_k, int window, float scale, void* stream_,
        const PagedArgs* paged = nullptr, bool noalloc = false) {
  constexpr int kKnown = ATTN_FWD_FP16 | ATTN_FWD_FP32 | ATTN_FWD_NONCAUSAL;
  if ((flags & ~kKnown) != 0) return ATTN_ERR_INVALID_ARG;
  if ((flags & ATTN_FWD_FP16) && (flags & ATTN_FWD_FP32)) return ATTN_ERR_INVALID_ARG;
  const bool causal = !(flags & ATTN_FWD_NONCAUSAL);
  if (!causal && window > 0) return ATTN_ERR_INVALID_ARG;
  const bool bf16 = !(flags & ATTN_FWD_FP32);  // a 16-bit type: the MFMA kernels
  attn_fwd_plan_t plan;
  const Geometry geo = device_geometry();
  int st = check_and_plan(B, Hq, Hkv, Q, K, D, Dv, window, scale, bf16, geo, &plan);
  if (st != ATTN_OK || plan.path == 0) return st;
  if (!q || !o || !lse) return ATTN_ERR_INVALID_ARG;
  if ((int64_t)B * Hkv * K > 0 && (!k || !v)) return ATTN_ERR_INVALID_ARG;
  if (paged && (int64_t)B * Hkv * K > 0 && !paged->block_table) return ATTN_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(o) || (k && !aligned16(k)) || (v && !aligned16(v)))
    return ATTN_ERR_INVALID_ARG;
  hipStream_t stream = static_cast<hipStream_t>(stream_);

  Params p = {};
  p.q = q; p.k = k; p.v = v; p.o = o; p.lse = lse; p.seqlens = seqlens_k;
  p.B = B; p.Hq = Hq; p.Hkv = Hkv; p.Q = Q; p.K = K; p.D = D; p.Dv = Dv;
  p.window = window > 0 ? window : 0;
  p.causal_shift = causal ? 0 : kNonCausalShift;
  p.f16 = (flags & ATTN_FWD_FP16) ? 1 : 0;
  p.group = Hq / Hkv;
  p.q_sign = scale < 0.f ? 1 : 0;
  // Kept strictly positive so a masked score (-inf) times it stays -inf; a
  // zero scale becomes 1e-30, which changes no weight: every finite score
  // times it rounds away against the reference max.
  p.scale_log2 = std::fmax(std::fabs(scale) * 1.4426950408889634f, 1e-30f);
  p.scale = scale;
  p.rows = p.group * Q;
  if (paged && K > 0) {
    p.block_table = paged->block_table;
    p.pages_per_seq = paged->pages_per_seq;
    p.page_shift = paged->page_shift;
    p.num_pages = paged->num_pages;
  }

  p.n_xcd = geo.xcds;
  p.n_split = 1;
  p.dv_parts = (D > 256 || Dv > 256) ? (Dv + 255) / 256 : 1;
  if (!bf16) return launch_status(launch_fwd_f32(p, stream));
  if (plan.path == 1 && plan.split_workers <= 1) return launch_status(launch_prefill_bf16(p, stream));

  // Split-KV decode or prefill: partial states in scratch (the stream's buffer,
  // or the library-held array for attn_fwd_noalloc).
  int64_t parts;
  if (plan.path == 1) {
    p.n_split = plan.split_workers;
    p.split_blocks = prefill_split_blocks(K, p.n_split);
    parts = (int64_t)plan.partial_slots * kPrefillBM;
  } else {
    p.n_workers = plan.split_workers;
    parts = (int64_t)plan.partial_slots * p.rows;
  }
  void* ws = nullptr;
  if (noalloc) {
    // Every partial slot the kernels read is written in the same call (a piece
    // with no key writes m = -inf), so the scratch needs no clearing.
    if (plan.workspace_bytes > kNoAllocScratchBytes) return ATTN_ERR_SCRATCH_LIMIT;
    if (parts > 0 && noalloc_scratch(&ws) != hipSuccess) {
      (void)hipGetLastError();
      return ATTN_ERR_HIP;
    }
  }
  ScratchCall call;  // held until the launches are enqueued (the allocating path only)
  if (!noalloc && parts > 0) {
    const int sst = call.acquire(stream, (size_t)plan.workspace_bytes, &ws);
    if (sst != ATTN_OK) return sst;
  }
  float* wsf = static_cast<float*>(ws);
  p.ws_acc = wsf;  // [parts][Dv] first: 16-byte aligned rows
  p.ws_m = wsf + parts * Dv;
  p.ws_l = p.ws_m + parts;
  const int launched = launch_status(plan.path == 1 ? launch_prefill_bf16(p, stream) : launch_decode_bf16(p, stream));
  const int recorded = call.record();
  return launched != ATTN_OK ? launched : recorded;
}

}  // namespace
}  // namespace attn

extern "C" {

int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq, int Hkv, int Q, int K,
             int D, int Dv, const int32_t* seqlens_k, int window, float scale, void* stream) {
  return attn::run(0, q, k, v, o, lse, B, Hq, Hkv, Q, K, D, Dv, seqlens_k, window, scale, stream);
}

int attn_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse, int B, int Hq, int Hkv, int Q,
                 int K, int D, int Dv, const int32_t* seqlens_k, int window, float scale, void* stream) {
  return attn::run(ATTN_FWD_FP32, q, k, v, o, lse, B, Hq, Hkv, Q, K, D, Dv, seqlens_k, window, scale, stream);
}

int attn_fwd_ex(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq, int Hkv, int Q,
                int K, int D, int Dv, const int32_t* seqlens_k, int window, float scale, int flags, void* stream) {
  return attn::run(flags, q, k, v, o, lse, B, Hq, Hkv, Q, K, D, Dv, seqlens_k, window, scale, stream);
}

int attn_fwd_noalloc(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq, int Hkv,
                     int Q, int K, int D, int Dv, const int32_t* seqlens_k, int window, float scale, int flags,
                     void* stream) {
  return attn::run(flags, q, k, v, o, lse, B, Hq, Hkv, Q, K, D, Dv, seqlens_k, window, scale, stream, nullptr, true);
}

int attn_fwd_paged(const void* q, const void* k_pages, const void* v_pages, void* o, float* lse, int B, int Hq,
                   int Hkv, int Q, int D, int Dv, const int32_t* block_table, int pages_per_seq, int page_size,
                   int num_pages, const int32_t* seqlens_k, int window, float scale, int flags, void* stream) {
  if (pages_per_seq < 0 || num_pages < 0 || page_size <= 0) return ATTN_ERR_INVALID_ARG;
  if ((page_size & (page_size - 1)) != 0 || page_size < (1 << attn::kMinPageShift) || page_size > (1 << 16))
    return ATTN_ERR_UNSUPPORTED;
  if (flags & ATTN_FWD_FP32) return ATTN_ERR_UNSUPPORTED;
  const int64_t K = (int64_t)pages_per_seq * page_size;
  if (K > INT32_MAX) return ATTN_ERR_UNSUPPORTED;
  if (K > 0 && num_pages == 0 && (int64_t)B * Hq * Q > 0) return ATTN_ERR_INVALID_ARG;
  int shift = 0;
  while ((1 << shift) < page_size) ++shift;
  const attn::PagedArgs pg{block_table, pages_per_seq, shift, num_pages};
  return attn::run(flags, q, k_pages, v_pages, o, lse, B, Hq, Hkv, Q, (int)K, D, Dv, seqlens_k, window, scale, stream,
                   &pg);
}

int attn_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout, void* dq,
             void* dk, void* dv, int B, int Hq, int Hkv, int Q, int K, int D, int Dv, const int32_t* seqlens_k,
             int window, float scale, int flags, void* stream_) {
  using namespace attn;
  constexpr int kKnown = ATTN_FWD_FP16 | ATTN_FWD_FP32 | ATTN_FWD_NONCAUSAL;
  if ((flags & ~kKnown) != 0) return ATTN_ERR_INVALID_ARG;
  if ((flags & ATTN_FWD_FP16) && (flags & ATTN_FWD_FP32)) return ATTN_ERR_INVALID_ARG;
  const bool causal = !(flags & ATTN_FWD_NONCAUSAL);
  if (!causal && window > 0) return ATTN_ERR_INVALID_ARG;
  if (B < 0 || Hq < 0 || Hkv < 0 || Q < 0 || K < 0 || D < 0 || Dv < 0) return ATTN_ERR_INVALID_ARG;
  if (Hq > 0 && (Hkv == 0 || Hq % Hkv != 0)) return ATTN_ERR_INVALID_ARG;
  if (!std::isfinite(scale)) return ATTN_ERR_INVALID_ARG;
  const int64_t rows = (int64_t)B * Hq * Q, keys = (int64_t)B * Hkv * K;
  if (rows == 0 && keys == 0) return ATTN_OK;
  if (flags & ATTN_FWD_FP32) return ATTN_ERR_UNSUPPORTED;
  auto width_ok = [](int d) { return d >= 16 && d <= 256 && d % 16 == 0; };
  if (!width_ok(D) || !width_ok(Dv)) return ATTN_ERR_UNSUPPORTED;
  const int64_t lim = (int64_t)1 << 31;
  if ((int64_t)Q * D * 2 >= lim || (int64_t)Q * Dv * 2 >= lim || (int64_t)K * D * 2 >= lim ||
      (int64_t)K * Dv * 2 >= lim)
    return ATTN_ERR_UNSUPPORTED;
  if ((int64_t)((Q + 127) / 128) * Hq * B > (int64_t)INT32_MAX || (int64_t)((K + 127) / 128) * Hkv * B > INT32_MAX ||
      (rows + 3) / 4 > (int64_t)INT32_MAX)
    return ATTN_ERR_UNSUPPORTED;
  if (keys > 0 && (!k || !v || !dk || !dv)) return ATTN_ERR_INVALID_ARG;
  if (rows > 0 && (!q || !o || !lse || !dout || !dq)) return ATTN_ERR_INVALID_ARG;
  for (const void* ptr : {q, k, v, o, dout, (const void*)dq, (const void*)dk, (const void*)dv})
    if (ptr && !aligned16(ptr)) return ATTN_ERR_INVALID_ARG;
  hipStream_t stream = static_cast<hipStream_t>(stream_);

  BwdParams p = {};
  p.q = q; p.k = k; p.v = v; p.o = o; p.dout = dout; p.lse = lse;
  p.dq = dq; p.dk = dk; p.dv = dv; p.seqlens = seqlens_k;
  p.B = B; p.Hq = Hq; p.Hkv = Hkv; p.Q = Q; p.K = K; p.D = D; p.Dv = Dv;
  p.window = window > 0 ? window : 0;
  p.causal_shift = causal ? 0 : kNonCausalShift;
  p.f16 = (flags & ATTN_FWD_FP16) ? 1 : 0;
  p.group = Hkv > 0 ? Hq / Hkv : 1;
  p.q_sign = scale < 0.f ? 1 : 0;
  p.scale_log2 = std::fmax(std::fabs(scale) * 1.4426950408889634f, 1e-30f);
  p.scale = scale;
  p.abs_scale = std::fabs(scale);

  // Scratch: delta and lse2 per row.
  void* ws = nullptr;
  ScratchCall call;
  if (rows > 0) {
    const int sst = call.acquire(stream, (size_t)(rows * 2 * 4), &ws);
    if (sst != ATTN_OK) return sst;
  }
  p.delta = static_cast<float*>(ws);
  p.lse2 = p.delta ? p.delta + rows : nullptr;
  const int launched = launch_status(launch_bwd_bf16(p, stream));
  const int recorded = call.record();
  return launched != ATTN_OK ? launched : recorded;
}

int attn_fwd_release_scratch(void) { return attn::release_stream_scratch(); }

const char* attn_fwd_strerror(int status) {
  switch (status) {
    case ATTN_OK: return "ok";
    case ATTN_ERR_INVALID_ARG: return "invalid argument";
    case ATTN_ERR_UNSUPPORTED:
      return "unsupported size (D and Dv must be multiples of 16 in [16, 512], [16, 128] in fp32)";
    case ATTN_ERR_OOM: return "scratch allocation failed";
    case ATTN_ERR_HIP: return "HIP launch or runtime error";
    case ATTN_ERR_SCRATCH_LIMIT:
      return "the call needs more split-KV scratch than attn_fwd_noalloc holds (64 MiB); use attn_fwd_ex";
    default: return "unknown status";
  }
}

int attn_fwd_plan(int B, int Hq, int Hkv, int Q, int K, int D, int Dv, int window, attn_fwd_plan_t* plan) {
  if (!plan) return ATTN_ERR_INVALID_ARG;
  return attn::check_and_plan(B, Hq, Hkv, Q, K, D, Dv, window, 1.0f, true, attn::device_geometry(), plan);
}

}  // extern "C"
