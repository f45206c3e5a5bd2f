// C ABI of libsdpa14: argument validation, stride resolution, the Philox
// state handed from forward to backward, launches and optional event timing.  The compute itself lives in fwd.hip / bwd.hip.
//
// The forward returns (out, lse, seed, offset) and the backward consumes
// (seed, offset), as in the sdpfa_fwd / sdpfa_bwd pair of the nvFuser PR "DID
// loop split for SDPA"; the RNG state travels from forward to backward instead
// of a stored mask (PyTorch PR "REDO of dropout support for mem eff", Summary).
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>

#include <algorithm>
#include <mutex>
#include <string>
#include <utility>
#include <vector>

#include "kernels.h"
#include "sdpa14.h"

using namespace sdpa14;

namespace {

thread_local std::string t_last_error;

std::mutex g_rng_mu;
uint64_t g_rng_seed = 0;
uint64_t g_rng_offset = 0;

constexpr int64_t kMaxSeq = int64_t(1) << 30;
constexpr int64_t kMaxGrid = (int64_t(1) << 31) - 1;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  t_last_error = buf;
  return code;
}

struct Desc {
  const uint16_t* ptr;
  int64_t B, H, S, E;
  Strides st;
  int dtype;
};

// Validates one tensor descriptor and resolves its strides.  Strides of
// size-1 dimensions never matter and are taken as 0.
int check_tensor(const sdpa_tensor* t, const char* name, Desc* d) {
  if (t == nullptr) return fail(SDPA_ERR_INVALID, "%s: descriptor is NULL", name);
  if (t->data == nullptr) return fail(SDPA_ERR_INVALID, "%s: data pointer is NULL", name);
  for (int i = 0; i < 4; ++i)
    if (t->size[i] < 1)
      return fail(SDPA_ERR_INVALID, "%s: size[%d] = %lld must be >= 1", name, i,
                  (long long)t->size[i]);
  if (t->dtype != SDPA_BF16 && t->dtype != SDPA_F16)
    return fail(SDPA_ERR_UNSUPPORTED, "%s: dtype %d is not supported (bf16 or f16)", name,
                t->dtype);
  if (t->stride[3] != 1 && t->size[3] > 1)
    return fail(SDPA_ERR_UNSUPPORTED, "%s: stride of the head dim is %lld, must be 1", name,
                (long long)t->stride[3]);
  int64_t st[3];
  for (int i = 0; i < 3; ++i) {
    st[i] = (t->size[i] == 1) ? 0 : t->stride[i];
    if (st[i] < 0)
      return fail(SDPA_ERR_UNSUPPORTED, "%s: negative stride[%d] is not supported", name, i);
    if (st[i] % 8 != 0)
      return fail(SDPA_ERR_UNSUPPORTED,
                  "%s: stride[%d] = %lld is not a multiple of 8 elements (16-byte rows)", name, i,
                  (long long)st[i]);
  }
  if (reinterpret_cast<uintptr_t>(t->data) % 16 != 0)
    return fail(SDPA_ERR_UNSUPPORTED, "%s: data pointer is not 16-byte aligned", name);
  if (t->size[2] > kMaxSeq) return fail(SDPA_ERR_UNSUPPORTED, "%s: sequence too long", name);
  if (t->size[0] * t->size[1] > kMaxGrid / 64)
    return fail(SDPA_ERR_UNSUPPORTED, "%s: batch*heads too large", name);
  d->ptr = static_cast<const uint16_t*>(t->data);
  d->B = t->size[0];
  d->H = t->size[1];
  d->S = t->size[2];
  d->E = t->size[3];
  d->st = Strides{st[0], st[1], st[2]};
  d->dtype = t->dtype;
  return SDPA_OK;
}

bool same_shape(const Desc& a, const Desc& b) {
  return a.B == b.B && a.H == b.H && a.S == b.S && a.E == b.E;
}

// Kernels address a (batch, head) slice with 32-bit byte offsets, including
// rows past S that tiles and trailing ring loads reach (fewer than 256; those
// read as zeros through the buffer range check).
bool slice_ok(const Desc& t) {
  return (t.S + 255) * t.st.s * 2 + t.E * 2 < (int64_t(1) << 31);
}

int check_qkv(const Desc& q, const Desc& k, const Desc& v) {
  if (q.B != k.B || q.B != v.B || q.H != k.H || q.H != v.H)
    return fail(SDPA_ERR_INVALID, "q, k, v disagree on batch or heads");
  if (k.S != v.S) return fail(SDPA_ERR_INVALID, "k and v have different key lengths");
  if (q.E != k.E) return fail(SDPA_ERR_INVALID, "q and k have different head dims");
  if (v.E != q.E) return fail(SDPA_ERR_INVALID, "value head dim Ev = %lld differs from E = %lld",
                              (long long)v.E, (long long)q.E);
  if (q.E % 8 != 0 || q.E > 128)
    return fail(SDPA_ERR_UNSUPPORTED,
                "head dim %lld is not supported (a multiple of 8, at most 128)", (long long)q.E);
  const int64_t grid_f = q.B * q.H * ((q.S + 31) / 32 + (k.S + 31) / 32);
  if (grid_f > kMaxGrid) return fail(SDPA_ERR_UNSUPPORTED, "problem too large for one launch");
  if (!slice_ok(q) || !slice_ok(k) || !slice_ok(v))
    return fail(SDPA_ERR_UNSUPPORTED, "a (batch, head) slice spans 2 GiB or more");
  return SDPA_OK;
}

// Byte span [lo, hi) that a buffer's elements occupy.
struct Span {
  uintptr_t lo, hi;
  const char* name;
};

Span tensor_span(const Desc& d, const char* name) {
  const int64_t last = (d.B - 1) * d.st.b + (d.H - 1) * d.st.h + (d.S - 1) * d.st.s + d.E;
  const uintptr_t lo = reinterpret_cast<uintptr_t>(d.ptr);
  return Span{lo, lo + (uintptr_t)last * 2u, name};
}

Span raw_span(const void* p, size_t bytes, const char* name) {
  const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
  return Span{lo, p == nullptr ? lo : lo + bytes, name};
}

// Every output span must be disjoint from every input span.  Outputs may share
// a buffer with one another (views of one packed tensor) unless `pairwise`;
// inputs may share anything.
int check_disjoint(const Span* outs, int n_out, const Span* ins, int n_in, bool pairwise) {
  for (int o = 0; o < n_out; ++o) {
    if (outs[o].lo == outs[o].hi) continue;
    for (int i = 0; i < n_in; ++i)
      if (ins[i].lo != ins[i].hi && outs[o].lo < ins[i].hi && ins[i].lo < outs[o].hi)
        return fail(SDPA_ERR_INVALID, "%s overlaps %s (outputs must not overlap inputs)",
                    outs[o].name, ins[i].name);
    for (int p = pairwise ? o + 1 : n_out; p < n_out; ++p)
      if (outs[p].lo != outs[p].hi && outs[o].lo < outs[p].hi && outs[p].lo < outs[o].hi)
        return fail(SDPA_ERR_INVALID, "%s overlaps %s", outs[o].name, outs[p].name);
  }
  return SDPA_OK;
}

int check_dropout(double p) {
  if (!(p >= 0.0 && p < 1.0)) return fail(SDPA_ERR_INVALID, "dropout_p = %g not in [0, 1)", p);
  return SDPA_OK;
}

int resolve_scale(double scale, int64_t E, float* out) {
  if (isnan(scale)) {
    *out = (float)(1.0 / sqrt((double)E));
    return SDPA_OK;
  }
  if (!(isfinite(scale) && scale > 0.0))
    return fail(SDPA_ERR_INVALID, "scale = %g must be finite and > 0 (NaN selects 1/sqrt(E))",
                scale);
  *out = (float)scale;
  return SDPA_OK;
}

DropoutParams make_dropout(double p, uint64_t seed, uint64_t offset, int64_t heads_total,
                           int64_t head_offset, const uint64_t* state) {
  DropoutParams d;
  d.offset = offset;
  d.seed_lo = (uint32_t)(seed & 0xFFFFFFFFu);
  d.seed_hi = (uint32_t)(seed >> 32);
  d.threshold = (uint32_t)floor(p * 4294967296.0);
  d.keep_scale = (float)(1.0 / (1.0 - p));
  d.heads_total = (int32_t)heads_total;
  d.head_offset = (int32_t)head_offset;
  d.state = state;
  return d;
}

// Resolved extension options of one call.
struct Ext {
  int64_t head_offset = 0;
  int64_t heads_total = 0;  // the call's H when not sharded
  uint64_t* rng_state = nullptr;
  uint64_t* rng_used = nullptr;
  const uint16_t* bias = nullptr;
  Strides sbias{0, 0, 0};
  uint32_t* keep_bits = nullptr;
  int bwd_parts = 3;  // bit 0: row pass, bit 1: main kernel
  uint16_t* dbias = nullptr;  // backward only
  Strides sdbias{0, 0, 0};
};

Span dbias_span(const Ext& e, int64_t B, int64_t H, int64_t Sq, int64_t Sk) {
  if (e.dbias == nullptr) return Span{0, 0, "dbias"};
  const int64_t last = (B - 1) * e.sdbias.b + (H - 1) * e.sdbias.h + (Sq - 1) * e.sdbias.s + Sk;
  const uintptr_t lo = reinterpret_cast<uintptr_t>(e.dbias);
  return Span{lo, lo + (uintptr_t)last * 2u, "dbias"};
}

Span bias_span(const Ext& e, int64_t B, int64_t H, int64_t Sq, int64_t Sk) {
  if (e.bias == nullptr) return Span{0, 0, "bias"};
  const int64_t last = (B - 1) * e.sbias.b + (H - 1) * e.sbias.h + (Sq - 1) * e.sbias.s + Sk;
  const uintptr_t lo = reinterpret_cast<uintptr_t>(e.bias);
  return Span{lo, lo + (uintptr_t)last * 2u, "bias"};
}

int check_bias(const sdpa_tensor* t, int64_t B, int64_t H, int64_t Sq, int64_t Sk, int dtype,
               Ext* e) {
  if (t->data == nullptr) return fail(SDPA_ERR_INVALID, "bias data is NULL");
  if (t->dtype != dtype)
    return fail(SDPA_ERR_UNSUPPORTED, "bias dtype must be the dtype of q");
  if (t->size[0] != B || t->size[1] != H || t->size[2] != Sq || t->size[3] != Sk)
    return fail(SDPA_ERR_INVALID, "bias must have logical shape [B, H, Sq, Sk] (stride 0 to broadcast)");
  if (t->stride[3] != 1) return fail(SDPA_ERR_UNSUPPORTED, "bias key stride must be 1");
  for (int i = 0; i < 3; ++i)
    if (t->stride[i] < 0 || t->stride[i] % 8 != 0)
      return fail(SDPA_ERR_UNSUPPORTED, "bias strides must be >= 0 and multiples of 8 elements");
  if (reinterpret_cast<uintptr_t>(t->data) % 16 != 0)
    return fail(SDPA_ERR_UNSUPPORTED, "bias data is not 16-byte aligned");
  if (((Sq + 128) * t->stride[2] + Sk) * 2 >= (int64_t(1) << 31))
    return fail(SDPA_ERR_UNSUPPORTED, "a (batch, head) slice of the bias spans 2 GiB or more");
  e->bias = static_cast<const uint16_t*>(t->data);
  e->sbias = Strides{t->stride[0], t->stride[1], t->stride[2]};
  return SDPA_OK;
}

// The bias gradient has one element per (b, h, i, j), written once each, so no
// two of its elements may share memory.
int check_dbias(const sdpa_tensor* t, int64_t B, int64_t H, int64_t Sq, int64_t Sk, int dtype,
                Ext* e) {
  if (t->data == nullptr) return fail(SDPA_ERR_INVALID, "dbias data is NULL");
  if (t->dtype != dtype) return fail(SDPA_ERR_UNSUPPORTED, "dbias dtype must be the dtype of q");
  if (t->size[0] != B || t->size[1] != H || t->size[2] != Sq || t->size[3] != Sk)
    return fail(SDPA_ERR_INVALID, "dbias must have logical shape [B, H, Sq, Sk]");
  if (t->stride[3] != 1) return fail(SDPA_ERR_UNSUPPORTED, "dbias key stride must be 1");
  for (int i = 0; i < 3; ++i)
    if (t->stride[i] < 1 || t->stride[i] % 8 != 0)
      return fail(SDPA_ERR_UNSUPPORTED, "dbias strides must be positive multiples of 8 elements");
  if (reinterpret_cast<uintptr_t>(t->data) % 16 != 0)
    return fail(SDPA_ERR_UNSUPPORTED, "dbias data is not 16-byte aligned");
  // Taken in order of stride, each dimension must step past everything the
  // dimensions below it span.
  struct Dim {
    int64_t n, s;
  } d[3] = {{B, t->stride[0]}, {H, t->stride[1]}, {Sq, t->stride[2]}};
  std::sort(d, d + 3, [](const Dim& a, const Dim& b) { return a.s < b.s; });
  int64_t extent = Sk;
  for (const Dim& x : d) {
    if (x.n == 1) continue;
    if (x.s < extent) return fail(SDPA_ERR_INVALID, "dbias elements overlap (strides too small)");
    extent = x.s * (x.n - 1) + extent;
  }
  if (((Sq - 1) * t->stride[2] + Sk) * 2 >= (int64_t(1) << 31))
    return fail(SDPA_ERR_UNSUPPORTED, "a (batch, head) slice of dbias spans 2 GiB or more");
  e->dbias = static_cast<uint16_t*>(t->data);
  e->sdbias = Strides{t->stride[0], t->stride[1], t->stride[2]};
  return SDPA_OK;
}

int check_ext(const sdpa_ext* ext, int64_t B, int64_t H, int64_t Sq, int64_t Sk, int dtype,
              bool forward, Ext* out) {
  Ext e;
  e.heads_total = H;
  if (ext != nullptr) {
    if (ext->head_offset < 0) return fail(SDPA_ERR_INVALID, "head_offset < 0");
    e.head_offset = ext->head_offset;
    e.heads_total = ext->heads_total == 0 ? H : ext->heads_total;
    if (e.heads_total < e.head_offset + H)
      return fail(SDPA_ERR_INVALID, "heads_total (%lld) < head_offset + H (%lld)",
                  (long long)e.heads_total, (long long)(e.head_offset + H));
    if (B * e.heads_total > kMaxGrid)
      return fail(SDPA_ERR_UNSUPPORTED, "B * heads_total too large");
    e.rng_state = forward ? ext->rng_state : nullptr;
    e.rng_used = ext->rng_used;
    if (forward && (e.rng_state == nullptr) != (e.rng_used == nullptr))
      return fail(SDPA_ERR_INVALID, "rng_state and rng_used go together");
    for (const uint64_t* ptr : {(const uint64_t*)e.rng_state, (const uint64_t*)e.rng_used})
      if (reinterpret_cast<uintptr_t>(ptr) % 8 != 0)
        return fail(SDPA_ERR_UNSUPPORTED, "device RNG buffers must be 8-byte aligned");
    if (e.rng_state != nullptr && e.rng_state == e.rng_used)
      return fail(SDPA_ERR_INVALID, "rng_state and rng_used must be distinct buffers");
    if (ext->bias != nullptr) {
      const int rc = check_bias(ext->bias, B, H, Sq, Sk, dtype, &e);
      if (rc) return rc;
    }
    e.keep_bits = ext->keep_bits;
    if (!forward) {
      if (ext->bwd_parts < 0 || ext->bwd_parts > 3)
        return fail(SDPA_ERR_INVALID, "bwd_parts = %d not in 0..3", ext->bwd_parts);
      e.bwd_parts = ext->bwd_parts == 0 ? 3 : ext->bwd_parts;
      if (ext->dbias != nullptr) {
        if (ext->bias == nullptr)
          return fail(SDPA_ERR_INVALID, "dbias needs a bias (the gradient is taken with respect to it)");
        const int rc = check_dbias(ext->dbias, B, H, Sq, Sk, dtype, &e);
        if (rc) return rc;
      }
    }
    if (reinterpret_cast<uintptr_t>(e.keep_bits) % 16 != 0)
      return fail(SDPA_ERR_UNSUPPORTED, "keep_bits is not 16-byte aligned");
    if (e.keep_bits != nullptr && Sq * keep_words(Sk) * 4 >= (int64_t(1) << 32))
      return fail(SDPA_ERR_UNSUPPORTED, "keep_bits of one (batch, head) span 4 GiB or more");
  }
  *out = e;
  return SDPA_OK;
}

uint64_t offset_advance(int64_t B, int64_t H, int64_t Sq, int64_t Sk) {
  return (uint64_t)B * (uint64_t)H * (uint64_t)Sq * (uint64_t)((Sk + 3) / 4);
}

// ---- event timing -----------------------------------------------------------
struct Profiler {
  std::mutex mu;
  bool on = false;
  std::vector<std::pair<hipEvent_t, hipEvent_t>> pool;
  std::vector<std::pair<hipEvent_t, hipEvent_t>> used[SDPA_KERNEL_KINDS];
};
Profiler g_prof;
constexpr size_t kMaxTimed = 8192;

template <typename F>
hipError_t timed_launch(int kind, hipStream_t stream, F launch) {
  std::pair<hipEvent_t, hipEvent_t> ev{nullptr, nullptr};
  {
    std::lock_guard<std::mutex> lk(g_prof.mu);
    if (g_prof.on && g_prof.used[kind].size() < kMaxTimed) {
      if (!g_prof.pool.empty()) {
        ev = g_prof.pool.back();
        g_prof.pool.pop_back();
      } else {
        if (hipEventCreate(&ev.first) != hipSuccess || hipEventCreate(&ev.second) != hipSuccess)
          ev = {nullptr, nullptr};
      }
    }
  }
  if (ev.first == nullptr) return launch();
  (void)hipEventRecord(ev.first, stream);
  const hipError_t err = launch();
  (void)hipEventRecord(ev.second, stream);
  std::lock_guard<std::mutex> lk(g_prof.mu);
  g_prof.used[kind].push_back(ev);
  return err;
}

int hip_status(hipError_t err, const char* what) {
  if (err == hipSuccess) return SDPA_OK;
  return fail(SDPA_ERR_HIP, "%s: %s", what, hipGetErrorString(err));
}

// SDPA14_FAIL_LAUNCH (set and not "0") makes every compute call fail as if
// the HIP runtime had refused its launch: the call returns SDPA_ERR_HIP
// before any HIP call, so error propagation can be tested without a GPU and
// without faulting one.  Read on every call.
bool forced_launch_failure(const char* what) {
  const char* s = getenv("SDPA14_FAIL_LAUNCH");
  if (s == nullptr || s[0] == '\0' || (s[0] == '0' && s[1] == '\0')) return false;
  fail(SDPA_ERR_HIP, "%s: launch failure forced by SDPA14_FAIL_LAUNCH; nothing was enqueued", what);
  return true;
}

// The forward workgroup shape is chosen per problem; SDPA14_FWD_SHAPE (1-4:
// four sub-tiles, two by two, one sub-tile with four key shares, the causal
// split launch) forces one, read on every call so that a process can compare
// them.  A shape the problem cannot take (3 at head dim 128, 4 without causal
// masking or at head dim 128) runs two by two.  SDPA14_BWD_ROLES (1: one
// launch, 2: two) does the same for the backward main pass; two launches need
// a call without dropout or bias, else it runs one.  SDPA14_BWD_ORDER=1 deals
// the backward's blocks in the order computed from the block index, which
// problems of more than 1024 key plus query blocks per head use, at any size.
// SDPA14_FWD_ORDER=1 runs the causal split forward in its default workgroup
// order, without the dispatch table that pairs long and short tiles.
TileChoice tile_choice() {
  TileChoice t{0, 0, 0, 0};
  if (const char* s = getenv("SDPA14_FWD_SHAPE")) t.fwd_shape = atoi(s);
  if (const char* s = getenv("SDPA14_BWD_ROLES")) t.bwd_roles = atoi(s);
  if (const char* s = getenv("SDPA14_BWD_ORDER")) t.bwd_order = atoi(s);
  if (const char* s = getenv("SDPA14_FWD_ORDER")) t.fwd_order = atoi(s);
  return t;
}

// ---- scratch of the allocation-free backward --------------------------------
// The row pass's two fp32 planes (-D and the base-2 LSE of every query row),
// 8 bytes per row, live in this array for sdpa_bwd_noalloc.  Each device holds
// its own copy until the process ends.  Host code never passes the array's
// name to a kernel: on the host it is only a stand-in for the symbol, and the
// device address comes from hipGetSymbolAddress, once per device, with that
// device current.
constexpr size_t kScratchBytes = size_t(4) << 20;  // 524288 query rows
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of this device's scratch (looked up on the first call per device).
int scratch_address(void** out) {
  int dev = -1;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return hip_status(err, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices)
    return fail(SDPA_ERR_UNSUPPORTED, "device %d is beyond the %d the library tracks", dev,
                kMaxDevices);
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    err = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (err != hipSuccess) return hip_status(err, "hipGetSymbolAddress(scratch)");
    if (ptr == nullptr || reinterpret_cast<uintptr_t>(ptr) % 256 != 0)
      return fail(SDPA_ERR_HIP, "scratch symbol has no usable device address");
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return SDPA_OK;
}

int bwd_call(const sdpa_tensor* dout, const sdpa_tensor* q, const sdpa_tensor* k,
             const sdpa_tensor* v, const sdpa_tensor* out, const float* lse, double dropout_p,
             int is_causal, uint64_t seed, uint64_t offset, double scale, const sdpa_tensor* dq,
             const sdpa_tensor* dk, const sdpa_tensor* dv, void* workspace,
             size_t workspace_bytes, bool use_scratch, const sdpa_ext* ext,
             sdpa_stream_t stream);

}  // namespace

extern "C" {

int sdpa_fwd(const sdpa_tensor* q, const sdpa_tensor* k, const sdpa_tensor* v,
             double dropout_p, int is_causal, double scale, const sdpa_tensor* out, float* lse,
             uint64_t* seed, uint64_t* offset, sdpa_stream_t stream) {
  if (lse == nullptr) return fail(SDPA_ERR_INVALID, "lse is NULL");
  return sdpa_fwd_ext(q, k, v, dropout_p, is_causal, scale, out, lse, seed, offset, nullptr,
                      stream);
}

int sdpa_fwd_ext(const sdpa_tensor* q, const sdpa_tensor* k, const sdpa_tensor* v,
                 double dropout_p, int is_causal, double scale, const sdpa_tensor* out,
                 float* lse, uint64_t* seed, uint64_t* offset, const sdpa_ext* ext,
                 sdpa_stream_t stream) {
  Desc dq, dk, dv, dout;
  int rc;
  if ((rc = check_tensor(q, "q", &dq))) return rc;
  if ((rc = check_tensor(k, "k", &dk))) return rc;
  if ((rc = check_tensor(v, "v", &dv))) return rc;
  if ((rc = check_tensor(out, "out", &dout))) return rc;
  if ((rc = check_qkv(dq, dk, dv))) return rc;
  if (!same_shape(dq, dout)) return fail(SDPA_ERR_INVALID, "out must have q's shape");
  // lse may be NULL here: an inference-only forward writes no log-sum-exp.
  if (reinterpret_cast<uintptr_t>(lse) % 4 != 0)
    return fail(SDPA_ERR_UNSUPPORTED, "lse is not 4-byte aligned");
  if ((rc = check_dropout(dropout_p))) return rc;
  float sc;
  if ((rc = resolve_scale(scale, dq.E, &sc))) return rc;
  Ext e;
  if (dk.dtype != dq.dtype || dv.dtype != dq.dtype || dout.dtype != dq.dtype)
    return fail(SDPA_ERR_INVALID, "q, k, v and out must share one dtype");
  if ((rc = check_ext(ext, dq.B, dq.H, dq.S, dk.S, dq.dtype, true, &e))) return rc;
  const bool drop = dropout_p > 0.0;
  {
    const Span outs[3] = {tensor_span(dout, "out"),
                          raw_span(lse, (size_t)(dq.B * dq.H * dq.S) * 4u, "lse"),
                          raw_span(drop ? e.keep_bits : nullptr,
                                   (size_t)(dq.B * dq.H * dq.S * keep_words(dk.S)) * 4u,
                                   "keep_bits")};
    const Span ins[4] = {tensor_span(dq, "q"), tensor_span(dk, "k"), tensor_span(dv, "v"),
                         bias_span(e, dq.B, dq.H, dq.S, dk.S)};
    if ((rc = check_disjoint(outs, 3, ins, 4, true))) return rc;
  }
  const uint64_t advance = offset_advance(dq.B, e.heads_total, dq.S, dk.S);
  const hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (forced_launch_failure("forward launch")) return SDPA_ERR_HIP;

  uint64_t s0 = 0, o0 = 0;
  if (e.rng_state == nullptr) {
    std::lock_guard<std::mutex> lk(g_rng_mu);
    s0 = g_rng_seed;
    o0 = g_rng_offset;
    if (drop) g_rng_offset += advance;
  }
  // A forward whose launch failed drew no bits: its advance is taken back
  // unless another call has moved the state since.
  auto undo_advance = [&] {
    if (!drop || e.rng_state != nullptr) return;
    std::lock_guard<std::mutex> lk(g_rng_mu);
    if (g_rng_seed == s0 && g_rng_offset == o0 + advance) g_rng_offset = o0;
  };
  if (e.rng_state == nullptr && seed) *seed = s0;
  if (e.rng_state == nullptr && offset) *offset = o0;
  (void)hipGetLastError();
  if (drop && e.rng_state != nullptr) {
    const hipError_t err = launch_rng_step(e.rng_state, e.rng_used, advance, st);
    if (err != hipSuccess) return hip_status(err, "RNG state launch");
  }

  FwdParams p;
  p.q = dq.ptr;
  p.k = dk.ptr;
  p.v = dv.ptr;
  p.o = const_cast<uint16_t*>(dout.ptr);
  p.lse = lse;
  p.sq = dq.st;
  p.sk = dk.st;
  p.sv = dv.st;
  p.so = dout.st;
  p.B = (int)dq.B;
  p.H = (int)dq.H;
  p.Sq = (int)dq.S;
  p.Sk = (int)dk.S;
  p.E = (int)dq.E;
  p.scale_log2 = sc * 1.44269504088896340736f;
  p.drop = make_dropout(dropout_p, s0, o0, e.heads_total, e.head_offset, e.rng_used);
  p.bias = e.bias;
  p.sbias = e.sbias;
  p.keep = drop ? e.keep_bits : nullptr;
  p.keep_w = keep_words(dk.S);
  const hipError_t err = timed_launch(SDPA_KERNEL_FWD, st, [&] {
    return launch_fwd(p, is_causal != 0, drop, dq.dtype == SDPA_F16, tile_choice(),
                      st);
  });
  if (err != hipSuccess) undo_advance();
  return hip_status(err, "forward launch");
}

int sdpa_bwd(const sdpa_tensor* dout, const sdpa_tensor* q, const sdpa_tensor* k,
             const sdpa_tensor* v, const sdpa_tensor* out, const float* lse, double dropout_p,
             int is_causal, uint64_t seed, uint64_t offset, double scale, const sdpa_tensor* dq,
             const sdpa_tensor* dk, const sdpa_tensor* dv, void* workspace,
             size_t workspace_bytes, sdpa_stream_t stream) {
  return sdpa_bwd_ext(dout, q, k, v, out, lse, dropout_p, is_causal, seed, offset, scale, dq, dk,
                      dv, workspace, workspace_bytes, nullptr, stream);
}

int sdpa_bwd_ext(const sdpa_tensor* dout, const sdpa_tensor* q, const sdpa_tensor* k,
                 const sdpa_tensor* v, const sdpa_tensor* out, const float* lse,
                 double dropout_p, int is_causal, uint64_t seed, uint64_t offset, double scale,
                 const sdpa_tensor* dq, const sdpa_tensor* dk, const sdpa_tensor* dv,
                 void* workspace, size_t workspace_bytes, const sdpa_ext* ext,
                 sdpa_stream_t stream) {
  return bwd_call(dout, q, k, v, out, lse, dropout_p, is_causal, seed, offset, scale, dq, dk, dv,
                  workspace, workspace_bytes, false, ext, stream);
}

int sdpa_bwd_noalloc(const sdpa_tensor* dout, const sdpa_tensor* q, const sdpa_tensor* k,
                     const sdpa_tensor* v, const sdpa_tensor* out, const float* lse,
                     double dropout_p, int is_causal, uint64_t seed, uint64_t offset,
                     double scale, const sdpa_tensor* dq, const sdpa_tensor* dk,
                     const sdpa_tensor* dv, const sdpa_ext* ext, sdpa_stream_t stream) {
  return bwd_call(dout, q, k, v, out, lse, dropout_p, is_causal, seed, offset, scale, dq, dk, dv,
                  nullptr, 0, true, ext, stream);
}

size_t sdpa_bwd_noalloc_max_rows(void) { return kScratchBytes / 8u; }

}  // extern "C"

namespace {

// The backward of sdpa_bwd_ext (workspace given by the caller) and of
// sdpa_bwd_noalloc (use_scratch: the library's device-resident scratch).
int bwd_call(const sdpa_tensor* dout, const sdpa_tensor* q, const sdpa_tensor* k,
             const sdpa_tensor* v, const sdpa_tensor* out, const float* lse, double dropout_p,
             int is_causal, uint64_t seed, uint64_t offset, double scale, const sdpa_tensor* dq,
             const sdpa_tensor* dk, const sdpa_tensor* dv, void* workspace,
             size_t workspace_bytes, bool use_scratch, const sdpa_ext* ext,
             sdpa_stream_t stream) {
  Desc ddo, dqi, dki, dvi, dout_i, dqo, dko, dvo;
  int rc;
  if ((rc = check_tensor(dout, "dout", &ddo))) return rc;
  if ((rc = check_tensor(q, "q", &dqi))) return rc;
  if ((rc = check_tensor(k, "k", &dki))) return rc;
  if ((rc = check_tensor(v, "v", &dvi))) return rc;
  if ((rc = check_tensor(out, "out", &dout_i))) return rc;
  if ((rc = check_tensor(dq, "dq", &dqo))) return rc;
  if ((rc = check_tensor(dk, "dk", &dko))) return rc;
  if ((rc = check_tensor(dv, "dv", &dvo))) return rc;
  if ((rc = check_qkv(dqi, dki, dvi))) return rc;
  if (!same_shape(dqi, ddo)) return fail(SDPA_ERR_INVALID, "dout must have q's shape");
  if (!same_shape(dqi, dout_i)) return fail(SDPA_ERR_INVALID, "out must have q's shape");
  if (!same_shape(dqi, dqo)) return fail(SDPA_ERR_INVALID, "dq must have q's shape");
  if (!same_shape(dki, dko)) return fail(SDPA_ERR_INVALID, "dk must have k's shape");
  if (!same_shape(dvi, dvo)) return fail(SDPA_ERR_INVALID, "dv must have v's shape");
  if (!slice_ok(ddo) || !slice_ok(dout_i))
    return fail(SDPA_ERR_UNSUPPORTED, "a (batch, head) slice spans 2 GiB or more");
  if (lse == nullptr) return fail(SDPA_ERR_INVALID, "lse is NULL");
  if (reinterpret_cast<uintptr_t>(lse) % 4 != 0)
    return fail(SDPA_ERR_UNSUPPORTED, "lse is not 4-byte aligned");
  if ((rc = check_dropout(dropout_p))) return rc;
  float sc;
  if ((rc = resolve_scale(scale, dqi.E, &sc))) return rc;
  if (use_scratch) {
    if (bwd_workspace_bytes(dqi.B, dqi.H, dqi.S) > kScratchBytes)
      return fail(SDPA_ERR_UNSUPPORTED,
                  "the allocation-free backward holds scratch for %zu query rows (B*H*Sq); "
                  "this call has %lld: use sdpa_bwd_ext with a workspace",
                  kScratchBytes / 8u, (long long)(dqi.B * dqi.H * dqi.S));
  } else {
    if (workspace == nullptr) return fail(SDPA_ERR_WORKSPACE, "workspace is NULL");
    if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0)
      return fail(SDPA_ERR_WORKSPACE, "workspace is not 256-byte aligned");
    if (workspace_bytes < bwd_workspace_bytes(dqi.B, dqi.H, dqi.S))
      return fail(SDPA_ERR_WORKSPACE, "workspace is smaller than sdpa_bwd_workspace_size()");
  }
  Ext e;
  for (const Desc* d : {&ddo, &dki, &dvi, &dout_i, &dqo, &dko, &dvo})
    if (d->dtype != dqi.dtype)
      return fail(SDPA_ERR_INVALID, "dout, q, k, v, out, dq, dk and dv must share one dtype");
  if ((rc = check_ext(ext, dqi.B, dqi.H, dqi.S, dki.S, dqi.dtype, false, &e))) return rc;
  {
    const int64_t rows = dqi.B * dqi.H * dqi.S;
    const Span outs[4] = {tensor_span(dqo, "dq"), tensor_span(dko, "dk"), tensor_span(dvo, "dv"),
                          raw_span(use_scratch ? nullptr : workspace,
                                   bwd_workspace_bytes(dqi.B, dqi.H, dqi.S), "workspace")};
    const Span ins[7] = {tensor_span(ddo, "dout"), tensor_span(dqi, "q"), tensor_span(dki, "k"),
                         tensor_span(dvi, "v"), tensor_span(dout_i, "out"),
                         raw_span(lse, (size_t)rows * 4u, "lse"),
                         bias_span(e, dqi.B, dqi.H, dqi.S, dki.S)};
    if ((rc = check_disjoint(outs, 4, ins, 7, false))) return rc;
    // The workspace may not share memory with the gradients either.
    if ((rc = check_disjoint(outs + 3, 1, outs, 3, false))) return rc;
    // Nor the bias gradient with any other argument.
    const Span db = dbias_span(e, dqi.B, dqi.H, dqi.S, dki.S);
    if ((rc = check_disjoint(&db, 1, ins, 7, false))) return rc;
    if ((rc = check_disjoint(&db, 1, outs, 4, false))) return rc;
  }

  BwdParams p;
  p.q = dqi.ptr;
  p.k = dki.ptr;
  p.v = dvi.ptr;
  p.o = dout_i.ptr;
  p.dout = ddo.ptr;
  p.dq = const_cast<uint16_t*>(dqo.ptr);
  p.dk = const_cast<uint16_t*>(dko.ptr);
  p.dv = const_cast<uint16_t*>(dvo.ptr);
  p.lse = lse;
  p.dl = static_cast<float*>(workspace);
  p.sq = dqi.st;
  p.sk = dki.st;
  p.sv = dvi.st;
  p.so = dout_i.st;
  p.sdo = ddo.st;
  p.sdq = dqo.st;
  p.sdk = dko.st;
  p.sdv = dvo.st;
  p.B = (int)dqi.B;
  p.H = (int)dqi.H;
  p.Sq = (int)dqi.S;
  p.Sk = (int)dki.S;
  p.E = (int)dqi.E;
  p.scale = sc;
  p.scale_log2 = sc * 1.44269504088896340736f;
  p.drop = make_dropout(dropout_p, seed, offset, e.heads_total, e.head_offset, e.rng_used);
  p.bias = e.bias;
  p.sbias = e.sbias;
  p.keep = dropout_p > 0.0 ? e.keep_bits : nullptr;
  p.keep_w = keep_words(dki.S);
  p.dbias = e.dbias;
  p.sdbias = e.sdbias;
  const bool causal = is_causal != 0, drop = dropout_p > 0.0;
  const hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (forced_launch_failure("backward launch")) return SDPA_ERR_HIP;
  if (use_scratch) {
    void* ptr = nullptr;
    if ((rc = scratch_address(&ptr))) return rc;
    p.dl = static_cast<float*>(ptr);
  }
  (void)hipGetLastError();
  const bool f16 = dqi.dtype == SDPA_F16;
  hipError_t err = hipSuccess;
  if (e.bwd_parts & 1)
    err = timed_launch(SDPA_KERNEL_BWD_ROWS, st, [&] { return launch_bwd_rows(p, f16, st); });
  if (err == hipSuccess && (e.bwd_parts & 2))
    err = timed_launch(SDPA_KERNEL_BWD, st,
                       [&] { return launch_bwd_main(p, causal, drop, f16, tile_choice(), st); });
  return hip_status(err, "backward launch");
}

}  // namespace

extern "C" {

size_t sdpa_keep_bits_size(int64_t B, int64_t H, int64_t Sq, int64_t Sk) {
  if (B <= 0 || H <= 0 || Sq <= 0 || Sk <= 0) return 0;
  return (size_t)B * (size_t)H * (size_t)Sq * (size_t)keep_words(Sk) * 4u;
}

size_t sdpa_bwd_workspace_size(int64_t B, int64_t H, int64_t Sq) {
  if (B <= 0 || H <= 0 || Sq <= 0) return 0;
  return bwd_workspace_bytes(B, H, Sq);
}

void sdpa_set_rng_state(uint64_t seed, uint64_t offset) {
  std::lock_guard<std::mutex> lk(g_rng_mu);
  g_rng_seed = seed;
  g_rng_offset = offset;
}

void sdpa_get_rng_state(uint64_t* seed, uint64_t* offset) {
  std::lock_guard<std::mutex> lk(g_rng_mu);
  if (seed) *seed = g_rng_seed;
  if (offset) *offset = g_rng_offset;
}

const char* sdpa_status_string(int status) {
  switch (status) {
    case SDPA_OK: return "SDPA_OK";
    case SDPA_ERR_INVALID: return "SDPA_ERR_INVALID";
    case SDPA_ERR_UNSUPPORTED: return "SDPA_ERR_UNSUPPORTED";
    case SDPA_ERR_WORKSPACE: return "SDPA_ERR_WORKSPACE";
    case SDPA_ERR_HIP: return "SDPA_ERR_HIP";
    default: return "SDPA_ERR_UNKNOWN";
  }
}

const char* sdpa_last_error(void) { return t_last_error.c_str(); }

int sdpa_debug_dropout_mask(uint64_t seed, uint64_t offset, double dropout_p, int64_t B,
                            int64_t H, int64_t Sq, int64_t Sk, uint8_t* mask,
                            sdpa_stream_t stream) {
  if (mask == nullptr) return fail(SDPA_ERR_INVALID, "mask is NULL");
  if (B < 1 || H < 1 || Sq < 1 || Sk < 1) return fail(SDPA_ERR_INVALID, "sizes must be >= 1");
  if (Sq > kMaxSeq || Sk > kMaxSeq || B * H > kMaxGrid / 64)
    return fail(SDPA_ERR_UNSUPPORTED, "problem too large");
  if (B * H * Sq * ((Sk + 3) / 4) / 256 > kMaxGrid)
    return fail(SDPA_ERR_UNSUPPORTED, "problem too large for one launch");
  int rc;
  if ((rc = check_dropout(dropout_p))) return rc;
  MaskParams p;
  p.mask = mask;
  p.B = (int)B;
  p.H = (int)H;
  p.Sq = (int)Sq;
  p.Sk = (int)Sk;
  p.drop = make_dropout(dropout_p, seed, offset, H, 0, nullptr);
  if (forced_launch_failure("mask launch")) return SDPA_ERR_HIP;
  (void)hipGetLastError();
  return hip_status(launch_mask(p, reinterpret_cast<hipStream_t>(stream)), "mask launch");
}

int sdpa_profile_enable(int on) {
  std::lock_guard<std::mutex> lk(g_prof.mu);
  g_prof.on = on != 0;
  return SDPA_OK;
}

int sdpa_profile_read(int kind, double* total_ms, int64_t* launches) {
  if (kind < 0 || kind >= SDPA_KERNEL_KINDS) return fail(SDPA_ERR_INVALID, "bad kernel kind");
  std::vector<std::pair<hipEvent_t, hipEvent_t>> evs;
  {
    std::lock_guard<std::mutex> lk(g_prof.mu);
    evs.swap(g_prof.used[kind]);
  }
  double sum = 0.0;
  int64_t n = 0;
  hipError_t first_err = hipSuccess;
  for (auto& ev : evs) {
    hipError_t err = hipEventSynchronize(ev.second);
    float ms = 0.f;
    if (err == hipSuccess) err = hipEventElapsedTime(&ms, ev.first, ev.second);
    if (err == hipSuccess) {
      sum += ms;
      ++n;
    } else if (first_err == hipSuccess) {
      first_err = err;
    }
  }
  {
    std::lock_guard<std::mutex> lk(g_prof.mu);
    for (auto& ev : evs) g_prof.pool.push_back(ev);
  }
  if (total_ms) *total_ms = sum;
  if (launches) *launches = n;
  return hip_status(first_err, "event timing");
}

}  // extern "C"
