// qdr_runtime.cpp -- host side of libqdr: argument checking, pool layout,
// device tables, kernel dispatch and the C ABI of include/qdr.h.
//
// The pool holds num_slots slots; each slot holds every head's packed block
// back to back at identical offsets (the precision allocation is fixed for
// all requests: review "STEPQuant: When and Where Errors Matter in Delta-Rule
// Recurrent State Quantization", Method).  (5B+1)-slot pools are the serving
// configuration accounted in the zhichai.net discussion of the paper.
#include "../../include/qdr.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <new>
#include <string>
#include <vector>

#include "qdr_internal.h"

namespace {

thread_local std::string g_err;

qdr_status fail(qdr_status st, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

qdr_status ok() {
  g_err.clear();
  return QDR_OK;
}

bool is_int_kind(int k) { return k == 2 || k == 4 || k == 6 || k == 8; }
bool is_kind(int k) { return is_int_kind(k) || k == 16 || k == 32; }
int kind_index(int k) {  // lists: INT2, INT4, INT6, INT8, FP16, FP32
  switch (k) {
    case 2: return 0;
    case 4: return 1;
    case 6: return 2;
    case 8: return 3;
    case 16: return 4;
    default: return 5;
  }
}

bool debug_slots() {
  const char *e = std::getenv("QDR_DEBUG");
  return e && e[0] == '1';
}

struct HostLayout {
  std::vector<uint64_t> head_off;
  std::vector<uint32_t> head_bytes, code_bytes;
  std::vector<uint8_t> words0, words1; // row units: words per column and half
  std::vector<qdr::RowProg> row_prog;  // row units: [H*128]
  std::vector<uint8_t> has_scales;
  uint64_t slot_stride = 0;
  int max_words = 0;
  int max_pivots = 0;                 // row units: most float rows in one half
  double stored_bits = 0;             // per slot
};

qdr_status check_desc(const qdr_pool_desc *d) {
  if (!d) return fail(QDR_E_INVAL, "desc is NULL");
  if (d->num_slots <= 0) return fail(QDR_E_INVAL, "num_slots must be > 0 (got %d)", d->num_slots);
  if (d->num_heads <= 0) return fail(QDR_E_INVAL, "num_heads must be > 0 (got %d)", d->num_heads);
  if (d->d_k != QDR_DIM || d->d_v != QDR_DIM)
    return fail(QDR_E_UNSUPPORTED, "d_k and d_v must be %d (got %d, %d)", QDR_DIM, d->d_k, d->d_v);
  if (d->unit != QDR_UNIT_HEAD && d->unit != QDR_UNIT_ROW) return fail(QDR_E_INVAL, "bad unit %d", d->unit);
  if (d->gate != QDR_GATE_SCALAR && d->gate != QDR_GATE_DIAG) return fail(QDR_E_INVAL, "bad gate %d", d->gate);
  if (d->scale_mode != QDR_SCALE_DUAL && d->scale_mode != QDR_SCALE_ROW_ABSMAX)
    return fail(QDR_E_INVAL, "bad scale_mode %d", d->scale_mode);
  if (d->fit_iters < 0 || d->fit_iters > 1) return fail(QDR_E_INVAL, "fit_iters must be 0 or 1");
  if (d->fit_iters > 0 && d->scale_mode != QDR_SCALE_DUAL)
    return fail(QDR_E_INVAL, "fit_iters requires dual-axis scales");
  if (d->scale_bits != 0 && d->scale_bits != 32 && d->scale_bits != 16)
    return fail(QDR_E_INVAL, "scale_bits must be 0, 32 or 16 (got %d)", d->scale_bits);
  if (!d->kinds) return fail(QDR_E_INVAL, "kinds is NULL");
  const int64_t nk = d->unit == QDR_UNIT_HEAD ? d->num_heads : (int64_t)d->num_heads * QDR_DIM;
  for (int64_t i = 0; i < nk; ++i)
    if (!is_kind(d->kinds[i])) return fail(QDR_E_INVAL, "kinds[%lld] = %d is not a kind", (long long)i, d->kinds[i]);
  if (d->scale_mode == QDR_SCALE_DUAL) {
    if (!d->omega) return fail(QDR_E_INVAL, "omega is NULL");
    const int64_t n = (int64_t)d->num_heads * QDR_DIM;
    for (int64_t i = 0; i < n; ++i) {
      const float w = d->omega[i];
      if (!(w >= 0x1p-40f && w <= 0x1p40f))
        return fail(QDR_E_INVAL, "omega[%lld] = %g outside [2^-40, 2^40]", (long long)i, (double)w);
    }
  }
  return QDR_OK;
}

// Block layout (see include/qdr.h): the code stream of a column holds rows
// 0..127 as b-bit fields; rows 0..63 and rows 64..127 each fill whole
// granules (16 B for whole-head units, 4 B for row units), granule g of
// column j at byte (g*128 + j)*G; then r (and c) when there are integer rows;
// blocks padded to 256 B.
void build_layout(const qdr_pool_desc *d, HostLayout &L) {
  const int H = d->num_heads;
  L.head_off.resize(H);
  L.head_bytes.resize(H);
  L.code_bytes.resize(H);
  L.words0.resize(H);
  L.words1.resize(H);
  L.has_scales.resize(H);
  if (d->unit == QDR_UNIT_ROW) {
    L.row_prog.resize((size_t)H * QDR_DIM);
  }
  uint64_t off = 0;
  double bits = 0;
  L.max_words = 0;
  L.max_pivots = 0;
  const uint64_t G = d->unit == QDR_UNIT_HEAD ? 16 : 4;
  for (int h = 0; h < H; ++h) {
    uint64_t ng = 0;
    bool any_int = false;
    for (int half = 0; half < 2; ++half) {
      uint64_t hbits = 0;
      int npiv = 0;
      for (int i = 64 * half; i < 64 * half + 64; ++i) {
        const int k = d->unit == QDR_UNIT_HEAD ? d->kinds[h] : d->kinds[(size_t)h * QDR_DIM + i];
        if (d->unit == QDR_UNIT_ROW) {
          const uint32_t x = (uint32_t)(hbits >> 5) * (QDR_DIM * 4u), y = (uint32_t)(hbits & 31u);
          const uint32_t wcode = k == 32 ? 0u : (uint32_t)k / 2u;
          const uint32_t completes = (k != 32 && y + (uint32_t)k >= 32u) ? qdr::kRowCompletes : 0u;
          L.row_prog[(size_t)h * QDR_DIM + i] = {x | (wcode << 5) | y | completes, (uint32_t)k};
        }
        hbits += (uint64_t)k;
        any_int = any_int || is_int_kind(k);
        npiv += is_int_kind(k) ? 0 : 1;
      }
      if (npiv > L.max_pivots) L.max_pivots = npiv;
      const uint64_t hg = (hbits + 8 * G - 1) / (8 * G);
      ng += hg;
      const int words = (int)(hg * G / 4);
      (half == 0 ? L.words0 : L.words1)[h] = (uint8_t)words;
      if (words > L.max_words) L.max_words = words;
    }
    const uint64_t code = ng * QDR_DIM * G;
    const uint64_t fb = d->scale_bits == 16 ? 2 : 4;   // bytes per stored factor
    const uint64_t scales = any_int ? (d->scale_mode == QDR_SCALE_DUAL ? 2 * QDR_DIM * fb : QDR_DIM * fb) : 0;
    const uint64_t blk = (code + scales + 255) / 256 * 256;
    L.head_off[h] = off;
    L.head_bytes[h] = (uint32_t)blk;
    L.code_bytes[h] = (uint32_t)code;
    L.has_scales[h] = any_int ? 1 : 0;
    off += blk;
    bits += 8.0 * (double)blk;
  }
  L.slot_stride = off;
  L.stored_bits = bits;
}

}  // namespace

struct qdr_pool {
  qdr_pool_desc desc{};
  std::vector<uint8_t> kinds;
  std::vector<float> omega;
  HostLayout L;
  qdr::PoolConfig cfg{};
  int device = 0;
  uint8_t *base = nullptr;
  bool owns_base = false;
  qdr::RowProg *d_row_prog = nullptr;
  float *d_omega = nullptr;
  uint32_t *d_err = nullptr;
  qdr::ListEntry *d_lists[qdr::kNumLists] = {};
  int32_t list_count[qdr::kNumLists] = {};
  // two-stream step: recorded on the write-back stream after its launches;
  // every later call on the pool orders its stream after it
  hipEvent_t wb_done = nullptr;
  bool wb_recorded = false;
  // whole-head pools with integer and float heads: the float-kind launches
  // run on a stream of the pool's own, forked from and joined back to the
  // caller's stream by two events, so they overlap the integer launch
  hipStream_t float_stream = nullptr;
  hipEvent_t fork_ev = nullptr, join_ev = nullptr;
};

namespace {

template <class T>
hipError_t upload(T **dst, const T *src, size_t n) {
  *dst = nullptr;
  if (n == 0) return hipSuccess;
  hipError_t e = hipMalloc(reinterpret_cast<void **>(dst), n * sizeof(T));
  if (e != hipSuccess) return e;
  return hipMemcpy(*dst, src, n * sizeof(T), hipMemcpyHostToDevice);
}

// Every integer head (lists 0..3, one per width), merged so that each width
// is spread evenly over the list: entry r of a width with n heads sits at
// position (r + 1/2) / n of the way through; ties keep width order.
std::vector<qdr::ListEntry> interleave_int_heads(const std::vector<std::vector<qdr::ListEntry>> &lists) {
  struct Key { double pos; int kind; qdr::ListEntry e; };
  std::vector<Key> keys;
  for (int k = 0; k < 4; ++k) {
    const size_t n = lists[k].size();
    for (size_t r = 0; r < n; ++r) keys.push_back({(r + 0.5) / (double)n, k, lists[k][r]});
  }
  std::stable_sort(keys.begin(), keys.end(), [](const Key &a, const Key &b) {
    return a.pos < b.pos || (a.pos == b.pos && a.kind < b.kind);
  });
  std::vector<qdr::ListEntry> out;
  out.reserve(keys.size());
  for (const Key &k : keys) out.push_back(k.e);
  return out;
}

void free_pool(qdr_pool *p) {
  if (!p) return;
  if (p->owns_base && p->base) (void)hipFree(p->base);
  (void)hipFree(p->d_row_prog);
  (void)hipFree(p->d_omega);
  (void)hipFree(p->d_err);
  for (auto &l : p->d_lists) (void)hipFree(l);
  if (p->wb_done) (void)hipEventDestroy(p->wb_done);
  if (p->fork_ev) (void)hipEventDestroy(p->fork_ev);
  if (p->join_ev) (void)hipEventDestroy(p->join_ev);
  if (p->float_stream) (void)hipStreamDestroy(p->float_stream);
  delete p;
}

qdr::LaunchArgs base_args(const qdr_pool *p) {
  qdr::LaunchArgs a{};
  a.pool = p->base;
  a.slot_stride = p->L.slot_stride;
  a.num_slots = p->desc.num_slots;
  a.H = p->desc.num_heads;
  a.row_prog = p->d_row_prog;
  a.omega = p->d_omega;
  a.err = p->d_err;
  return a;
}

qdr_status check_slots_host(const qdr_pool *p, const int32_t *slots, int32_t n, hipStream_t st,
                            bool allow_padding) {
  if (!debug_slots()) return QDR_OK;
  std::vector<int32_t> h(n);
  if (hipMemcpyAsync(h.data(), slots, sizeof(int32_t) * n, hipMemcpyDeviceToHost, st) != hipSuccess ||
      hipStreamSynchronize(st) != hipSuccess)
    return fail(QDR_E_DEVICE, "QDR_DEBUG: cannot read the slot table");
  std::vector<uint8_t> seen(p->desc.num_slots, 0);
  for (int32_t i = 0; i < n; ++i) {
    const int32_t s = h[i];
    if (s == -1 && allow_padding) continue;
    if (s < 0 || s >= p->desc.num_slots) return fail(QDR_E_SLOT, "QDR_DEBUG: slots[%d] = %d out of range", i, s);
    if (seen[s]) return fail(QDR_E_SLOT, "QDR_DEBUG: slot %d listed twice", s);
    seen[s] = 1;
  }
  return QDR_OK;
}

// Order `st` after the last two-stream write-back on this pool (a no-op when
// there has been none; waiting on a completed event costs nothing).
hipError_t after_writeback(qdr_pool *p, hipStream_t st) {
  if (!p->wb_recorded) return hipSuccess;
  return hipStreamWaitEvent(st, p->wb_done, 0);
}

qdr_status dispatch(qdr_pool *p, qdr::LaunchArgs a, int n, int mode, hipStream_t st) {
  const hipError_t we = after_writeback(p, st);
  if (we != hipSuccess) return fail(QDR_E_DEVICE, "stream wait failed: %s", hipGetErrorString(we));
  const qdr::ListEntry *lists[qdr::kNumLists];
  for (int i = 0; i < qdr::kNumLists; ++i) lists[i] = p->d_lists[i];
  hipError_t e;
  if (p->float_stream && n > 0) {
    // fork: the float stream starts after everything before this call on
    // st; join: st continues after the float launches
    e = hipEventRecord(p->fork_ev, st);
    if (e == hipSuccess) e = hipStreamWaitEvent(p->float_stream, p->fork_ev, 0);
    if (e == hipSuccess) e = qdr::launch_all(p->cfg, a, n, lists, p->list_count, mode, st, p->float_stream);
    if (e == hipSuccess) e = hipEventRecord(p->join_ev, p->float_stream);
    if (e == hipSuccess) e = hipStreamWaitEvent(st, p->join_ev, 0);
  } else {
    e = qdr::launch_all(p->cfg, a, n, lists, p->list_count, mode, st, st);
  }
  if (e == hipErrorNotSupported) return fail(QDR_E_UNSUPPORTED, "this pool configuration has no kernel");
  if (e != hipSuccess) return fail(QDR_E_DEVICE, "kernel launch failed: %s", hipGetErrorString(e));
  return ok();
}

}  // namespace

extern "C" {

qdr_status qdr_pool_bytes(const qdr_pool_desc *desc, size_t *bytes) {
  qdr_status st = check_desc(desc);
  if (st != QDR_OK) return st;
  if (!bytes) return fail(QDR_E_INVAL, "bytes is NULL");
  HostLayout L;
  build_layout(desc, L);
  *bytes = (size_t)(L.slot_stride * (uint64_t)desc->num_slots);
  return ok();
}

qdr_status qdr_pool_create(const qdr_pool_desc *desc, void *dev_mem, size_t dev_bytes, qdr_pool **out) {
  qdr_status st = check_desc(desc);
  if (st != QDR_OK) return st;
  if (!out) return fail(QDR_E_INVAL, "out is NULL");
  *out = nullptr;
  qdr_pool *p = new (std::nothrow) qdr_pool();
  if (!p) return fail(QDR_E_NOMEM, "host allocation failed");
  p->desc = *desc;
  const size_t nk = desc->unit == QDR_UNIT_HEAD ? desc->num_heads : (size_t)desc->num_heads * QDR_DIM;
  p->kinds.assign(desc->kinds, desc->kinds + nk);
  p->omega.assign((size_t)desc->num_heads * QDR_DIM, 1.0f);
  if (desc->omega) std::memcpy(p->omega.data(), desc->omega, sizeof(float) * p->omega.size());
  p->desc.kinds = p->kinds.data();
  p->desc.omega = p->omega.data();
  build_layout(&p->desc, p->L);
  p->cfg.unit = desc->unit;
  p->cfg.gate = desc->gate;
  p->cfg.scale_mode = desc->scale_mode;
  p->cfg.fit_iters = desc->fit_iters;
  p->cfg.scale_bits = desc->scale_bits == 16 ? 16 : 32;
  p->cfg.max_words = p->L.max_words;
  p->cfg.max_pivots = p->L.max_pivots;
  if (hipGetDevice(&p->device) != hipSuccess) { free_pool(p); return fail(QDR_E_DEVICE, "no HIP device"); }

  const uint64_t total = p->L.slot_stride * (uint64_t)desc->num_slots;
  if (dev_mem) {
    if (dev_bytes < total) { free_pool(p); return fail(QDR_E_NOMEM, "dev_mem holds %zu bytes, pool needs %llu", dev_bytes, (unsigned long long)total); }
    if (reinterpret_cast<uintptr_t>(dev_mem) % 256) { free_pool(p); return fail(QDR_E_INVAL, "dev_mem must be 256-byte aligned"); }
    p->base = static_cast<uint8_t *>(dev_mem);
  } else {
    if (hipMalloc(reinterpret_cast<void **>(&p->base), total) != hipSuccess) {
      (void)hipGetLastError();
      p->base = nullptr;
      free_pool(p);
      return fail(QDR_E_NOMEM, "hipMalloc of %llu bytes failed", (unsigned long long)total);
    }
    p->owns_base = true;
  }
  std::vector<qdr::HeadInfo> hi(desc->num_heads);
  std::vector<std::vector<qdr::ListEntry>> lists(qdr::kNumLists);
  for (int h = 0; h < desc->num_heads; ++h) {
    hi[h].off = p->L.head_off[h];
    hi[h].code_bytes = p->L.code_bytes[h];
    hi[h].words0 = p->L.words0[h];
    hi[h].words1 = p->L.words1[h];
    hi[h].kind = desc->unit == QDR_UNIT_HEAD ? p->kinds[h] : 0;
    hi[h].has_scales = p->L.has_scales[h];
    qdr::ListEntry le{};
    le.info = hi[h];
    le.h = h;
    if (desc->unit == QDR_UNIT_HEAD) lists[kind_index(p->kinds[h])].push_back(le);
    else lists[0].push_back(le);
  }
  if (desc->unit == QDR_UNIT_HEAD) lists[qdr::kListIntMix] = interleave_int_heads(lists);
  hipError_t e = hipMemset(p->base, 0, total);
  if (e == hipSuccess) e = upload(&p->d_omega, p->omega.data(), p->omega.size());
  if (e == hipSuccess && desc->unit == QDR_UNIT_ROW) {
    e = upload(&p->d_row_prog, p->L.row_prog.data(), p->L.row_prog.size());
  }
  for (int i = 0; i < qdr::kNumLists && e == hipSuccess; ++i) {
    p->list_count[i] = (int32_t)lists[i].size();
    e = upload(&p->d_lists[i], lists[i].data(), lists[i].size());
  }
  const bool has_int_heads = p->list_count[qdr::kListIntMix] > 0;
  const bool has_float_heads = desc->unit == QDR_UNIT_HEAD && (p->list_count[4] > 0 || p->list_count[5] > 0);
  if (e == hipSuccess && has_int_heads && has_float_heads) {
    e = hipStreamCreateWithFlags(&p->float_stream, hipStreamNonBlocking);   // default priority
    if (e == hipSuccess) e = hipEventCreateWithFlags(&p->fork_ev, hipEventDisableTiming);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&p->join_ev, hipEventDisableTiming);
  }
  if (e == hipSuccess) e = hipMalloc(reinterpret_cast<void **>(&p->d_err), sizeof(uint32_t));
  if (e == hipSuccess) e = hipMemset(p->d_err, 0, sizeof(uint32_t));
  if (e == hipSuccess) e = hipDeviceSynchronize();
  if (e != hipSuccess) {
    (void)hipGetLastError();
    free_pool(p);
    return fail(e == hipErrorOutOfMemory ? QDR_E_NOMEM : QDR_E_DEVICE, "pool setup failed: %s", hipGetErrorString(e));
  }
  *out = p;
  return ok();
}

qdr_status qdr_pool_destroy(qdr_pool *pool) {
  if (!pool) return ok();
  (void)hipDeviceSynchronize();
  free_pool(pool);
  return ok();
}

static qdr_status simple_mode(qdr_pool *pool, const int32_t *slots, int32_t n, const float *S_in, float *S_out,
                              int mode, void *stream) {
  if (!pool) return fail(QDR_E_INVAL, "pool is NULL");
  if (n < 0) return fail(QDR_E_INVAL, "n must be >= 0");
  if (n == 0) return ok();
  if (!slots) return fail(QDR_E_INVAL, "slots is NULL");
  if (mode == qdr::MODE_PACK && !S_in) return fail(QDR_E_INVAL, "S is NULL");
  if (mode == qdr::MODE_UNPACK && !S_out) return fail(QDR_E_INVAL, "S_out is NULL");
  hipStream_t st = static_cast<hipStream_t>(stream);
  qdr_status cs = check_slots_host(pool, slots, n, st, mode == qdr::MODE_UNPACK);
  if (cs != QDR_OK) return cs;
  qdr::LaunchArgs a = base_args(pool);
  a.slots = slots;
  a.S_in = S_in;
  a.S_out = S_out;
  return dispatch(pool, a, n, mode, st);
}

qdr_status qdr_slot_reset(qdr_pool *pool, const int32_t *slots, int32_t n, void *stream) {
  return simple_mode(pool, slots, n, nullptr, nullptr, qdr::MODE_RESET, stream);
}

qdr_status qdr_pack(qdr_pool *pool, const int32_t *slots, int32_t n, const float *S, void *stream) {
  return simple_mode(pool, slots, n, S, nullptr, qdr::MODE_PACK, stream);
}

qdr_status qdr_unpack(qdr_pool *pool, const int32_t *slots, int32_t n, float *S_out, void *stream) {
  return simple_mode(pool, slots, n, nullptr, S_out, qdr::MODE_UNPACK, stream);
}

qdr_status qdr_decode_step(qdr_pool *pool, const int32_t *slots, int32_t B, const float *q, const float *k,
                           const float *v, const float *beta, const float *gate, float *o, void *stream) {
  if (!pool) return fail(QDR_E_INVAL, "pool is NULL");
  if (B < 0) return fail(QDR_E_INVAL, "B must be >= 0");
  if (B == 0) return ok();
  if (!slots || !q || !k || !v || !beta || !gate || !o)
    return fail(QDR_E_INVAL, "a tensor pointer is NULL");
  hipStream_t st = static_cast<hipStream_t>(stream);
  qdr_status cs = check_slots_host(pool, slots, B, st, true);
  if (cs != QDR_OK) return cs;
  qdr::LaunchArgs a = base_args(pool);
  a.slots = slots;
  a.q = q;
  a.k = k;
  a.v = v;
  a.beta = beta;
  a.gate = gate;
  a.o = o;
  return dispatch(pool, a, B, qdr::MODE_STEP, st);
}

qdr_status qdr_decode_step_bf16(qdr_pool *pool, const int32_t *slots, int32_t B, const uint16_t *q,
                                const uint16_t *k, const uint16_t *v, const float *beta, const float *gate,
                                uint16_t *o, void *stream) {
  if (!pool) return fail(QDR_E_INVAL, "pool is NULL");
  if (B < 0) return fail(QDR_E_INVAL, "B must be >= 0");
  if (B == 0) return ok();
  if (!slots || !q || !k || !v || !beta || !gate || !o)
    return fail(QDR_E_INVAL, "a tensor pointer is NULL");
  hipStream_t st = static_cast<hipStream_t>(stream);
  qdr_status cs = check_slots_host(pool, slots, B, st, true);
  if (cs != QDR_OK) return cs;
  qdr::LaunchArgs a = base_args(pool);
  a.slots = slots;
  a.q = reinterpret_cast<const float *>(q);
  a.k = reinterpret_cast<const float *>(k);
  a.v = reinterpret_cast<const float *>(v);
  a.beta = beta;
  a.gate = gate;
  a.o = reinterpret_cast<float *>(o);
  return dispatch(pool, a, B, qdr::MODE_STEP_BF16, st);
}

qdr_status qdr_decode_step_split(qdr_pool *pool, const int32_t *slots, int32_t B, const float *q, const float *k,
                                 const float *v, const float *beta, const float *gate, float *o,
                                 void *stream_readout, void *stream_writeback) {
  if (!pool) return fail(QDR_E_INVAL, "pool is NULL");
  if (B < 0) return fail(QDR_E_INVAL, "B must be >= 0");
  if (B == 0) return ok();
  if (!slots || !q || !k || !v || !beta || !gate || !o)
    return fail(QDR_E_INVAL, "a tensor pointer is NULL");
  hipStream_t sr = static_cast<hipStream_t>(stream_readout);
  hipStream_t sw = static_cast<hipStream_t>(stream_writeback);
  qdr_status cs = check_slots_host(pool, slots, B, sr, true);
  if (cs != QDR_OK) return cs;
  if (!pool->wb_done) {
    const hipError_t e = hipEventCreateWithFlags(&pool->wb_done, hipEventDisableTiming);
    if (e != hipSuccess) {
      pool->wb_done = nullptr;
      return fail(QDR_E_DEVICE, "event create failed: %s", hipGetErrorString(e));
    }
  }
  qdr::LaunchArgs a = base_args(pool);
  a.slots = slots;
  a.q = q;
  a.k = k;
  a.v = v;
  a.beta = beta;
  a.gate = gate;
  a.o = o;
  // 1. readout-first launches on stream_readout (ordered after any earlier write-back)
  qdr_status st = dispatch(pool, a, B, qdr::MODE_READOUT, sr);
  if (st != QDR_OK) return st;
  // 2. the write-back launches on stream_writeback, after the readout has read
  //    the codes they overwrite; the full step without the o store
  hipError_t e = hipEventRecord(pool->wb_done, sr);
  if (e == hipSuccess) e = hipStreamWaitEvent(sw, pool->wb_done, 0);
  if (e != hipSuccess) return fail(QDR_E_DEVICE, "stream ordering failed: %s", hipGetErrorString(e));
  a.o = nullptr;
  st = dispatch(pool, a, B, qdr::MODE_WRITEBACK, sw);
  if (st != QDR_OK) return st;
  // 3. later calls on this pool, on any stream, wait for the write-back
  e = hipEventRecord(pool->wb_done, sw);
  if (e != hipSuccess) return fail(QDR_E_DEVICE, "event record failed: %s", hipGetErrorString(e));
  pool->wb_recorded = true;
  return ok();
}

qdr_status qdr_get_layout(const qdr_pool *pool, qdr_layout *out) {
  if (!pool || !out) return fail(QDR_E_INVAL, "pool or out is NULL");
  out->slot_stride = pool->L.slot_stride;
  out->total_bytes = pool->L.slot_stride * (uint64_t)pool->desc.num_slots;
  out->num_slots = pool->desc.num_slots;
  out->num_heads = pool->desc.num_heads;
  out->head_off = pool->L.head_off.data();
  out->head_bytes = pool->L.head_bytes.data();
  out->code_bytes = pool->L.code_bytes.data();
  out->base = pool->base;
  out->bits_per_value = pool->L.stored_bits / ((double)pool->desc.num_heads * QDR_DIM * QDR_DIM);
  return ok();
}

qdr_status qdr_read_raw(qdr_pool *pool, int32_t slot, void *host_dst, size_t n, void *stream) {
  if (!pool || !host_dst) return fail(QDR_E_INVAL, "pool or host_dst is NULL");
  if (slot < 0 || slot >= pool->desc.num_slots) return fail(QDR_E_SLOT, "slot %d out of range", slot);
  if (n != pool->L.slot_stride) return fail(QDR_E_INVAL, "n must equal slot_stride (%llu)", (unsigned long long)pool->L.slot_stride);
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e = after_writeback(pool, st);
  if (e == hipSuccess) e = hipMemcpyAsync(host_dst, pool->base + (size_t)slot * pool->L.slot_stride, n, hipMemcpyDeviceToHost, st);
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  if (e != hipSuccess) return fail(QDR_E_DEVICE, "read_raw: %s", hipGetErrorString(e));
  return ok();
}

qdr_status qdr_write_raw(qdr_pool *pool, int32_t slot, const void *host_src, size_t n, void *stream) {
  if (!pool || !host_src) return fail(QDR_E_INVAL, "pool or host_src is NULL");
  if (slot < 0 || slot >= pool->desc.num_slots) return fail(QDR_E_SLOT, "slot %d out of range", slot);
  if (n != pool->L.slot_stride) return fail(QDR_E_INVAL, "n must equal slot_stride (%llu)", (unsigned long long)pool->L.slot_stride);
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e = after_writeback(pool, st);
  if (e == hipSuccess) e = hipMemcpyAsync(pool->base + (size_t)slot * pool->L.slot_stride, host_src, n, hipMemcpyHostToDevice, st);
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  if (e != hipSuccess) return fail(QDR_E_DEVICE, "write_raw: %s", hipGetErrorString(e));
  return ok();
}

qdr_status qdr_poll_device_error(qdr_pool *pool, uint32_t *flags) {
  if (!pool || !flags) return fail(QDR_E_INVAL, "pool or flags is NULL");
  hipError_t e = hipDeviceSynchronize();
  if (e == hipSuccess) e = hipMemcpy(flags, pool->d_err, sizeof(uint32_t), hipMemcpyDeviceToHost);
  if (e == hipSuccess) e = hipMemset(pool->d_err, 0, sizeof(uint32_t));
  if (e == hipSuccess) e = hipDeviceSynchronize();
  if (e != hipSuccess) return fail(QDR_E_DEVICE, "poll_device_error: %s", hipGetErrorString(e));
  return ok();
}

const char *qdr_last_error(void) { return g_err.c_str(); }

}  // extern "C"
