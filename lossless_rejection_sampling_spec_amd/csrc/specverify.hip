// specverify.hip -- HIP kernels and C ABI of the batched speculative-decoding
// verify (see include/specverify.h for the contract of every entry point).
//
// Written for MI355X (gfx950): wave64, 256-thread workgroups, 128-bit global
// loads, NaN-propagating 3-input max, no matrix cores (the verify is a
// bandwidth-bound stream over vocabulary rows).
//
// One fused kernel, k_verify, does the whole verify of a batch:
//   draft       (sampled calls with draft rows) launched first: workgroup
//   strips      (b, j, s) reads a strip of S chunks of draft row j of a
//               draft-logit request once from HBM and publishes per-chunk
//               statistics (max, sum of exp2 terms).
//   producers   workgroup (b, j, s) reads a strip of S chunks (CHUNK elements
//               each) of target row j of request b once from HBM and
//               publishes per-chunk statistics (max, sum of exp2 terms, or
//               argmax) and the values at the draft id.
//   finalizer   the last producer of a request in launch order waits for the
//               request's statistics, merges them in a fixed order, runs the
//               acceptance scan as a 64-lane ballot (lane j = position j),
//               writes the outputs, and draws the final token itself when that
//               needs only the target row (bonus draw, one-hot draft
//               rejection); greedy requests end here.
//   helpers     nc workgroups per logit/probability-draft request, launched
//               after every producer of the call: when the
//               finalizer reports a rejection they compute the residual mass
//               max(0, p - q) of one chunk each and exchange the masses; the
//               helper whose chunk holds u * W draws the token from the
//               registers it holds (for rows of more than 32 chunks the last
//               helper gathers the masses, re-reads the chosen chunk and draws).
// k_thresh (only when top-k / top-p arrays are given) runs first and computes
// each filtered row's raw-logit threshold tau (kept iff l >= tau).
//
// Hand-off between workgroups.  Every value one workgroup passes to another
// travels in a 64-bit word whose top bit is a "fresh" tag: the writer stores
// the word with one agent-scope atomic store (coherent across the eight XCD
// L2 caches, no fence, no counter), the single reader of that word waits for
// the tag, takes the payload and stores the word back without its tag.
// Draft strips and producers wait for nothing; finalizers wait for draft
// strips and producers launched before them; helpers wait for their finalizer and for the other helpers of the
// same request, which are launched together (see helper()).  Every wait is
// bounded (a request whose wait runs out reports SV_ROW_INTERNAL).  A
// workspace is therefore left with no tag set when a call ends.
//
// Numerics (temperature T, c = log2(e)/T rounded to fp32; every fp64 step
// uses that same c, so all terms share one temperature):
//   element term    in fp32 against a reference r >= l: in the producers
//                   exp2(l*c - m*c) with r = m the thread's own max, m*c
//                   rounded once and the argument formed by one fused
//                   multiply-add; in the finalizer and the helpers
//                   exp2((l - r) * c) with r the chunk max.
//   chunk sum       s_c = sum over threads of (fp32 sum of the thread's terms)
//                   * exp2((m_t - m_c) * c), rescaled and added in fp64 and
//                   published as fp32 with the chunk max m_c.
//   chunk merge     S = sum_c s_c * exp2((m_c - M) * c) in fp64: 16 lanes per
//                   row take chunks c = lane, lane + 16, ... in order, then a
//                   fixed butterfly adds the 16 partial sums.
//   gathered p(x)   exp2((l_x - M) * c) / S in fp64; acceptance u*q(x) < p(x)
//                   in fp64.
//   final draw      per-element weights in fp64; a chunk's mass is the total
//                   of an fp64 block scan of its segment sums, exchanged
//                   between helpers rounded to fp32; sequential prefix over
//                   chunks in fp64, then the scan inside the chosen chunk in
//                   token order.

#include <hip/hip_runtime.h>
#include <float.h>
#include <stdint.h>

#include <algorithm>
#include <cmath>
#include <mutex>
#include <type_traits>

#include "specverify.h"

namespace sv {

constexpr int WG = 256;
constexpr int NWAVE = WG / 64;
constexpr int CHUNK = 8192;
constexpr int EPT = CHUNK / WG;   // elements per thread per chunk
constexpr int MAX_NC = 512;       // chunks per row (vocab <= 4,194,304)
constexpr int MAX_K = 63;         // k+1 positions fit one wave
constexpr int STAGE_MAX = 49152;  // bytes of LDS the finalizer may stage statistics in
#ifndef SV_SPIN_MAX
#define SV_SPIN_MAX (1 << 18)
#endif
constexpr int SPIN_MAX = SV_SPIN_MAX;  // polls before a wait gives up
constexpr float NEG_INF = -__builtin_inff();
constexpr float POS_INF = __builtin_inff();
constexpr double LOG2E = 1.4426950408889634;
constexpr uint32_t TAG = 0x80000000u;     // "fresh" bit of a hand-off word (high half)
// high half of a threshold word: the threshold kernel published the row's
// statistics itself (the row's producers have nothing to do)
constexpr uint32_t THR_PUBLISHED = 1u;
constexpr uint32_t F_NONE = 0x40000000u;  // helper decision: no residual to compute
constexpr uint32_t F_BAD = 0x20000000u;   // residual chunk saw an invalid probability
// Words of one helper's decision record: 0 the target chunk max (the stop
// position a in the flag bits), 1 the draft chunk max, 2-3 and 4-5 the fp64
// target and draft normalizers, 6-7 the target and draft row maxima.
constexpr int DEC_W = 8;
// Up to this many chunks per row, the helpers of a request exchange their
// residual masses (nc * nc words per request); beyond, the last one gathers.
constexpr int PEER_MAX = 32;

typedef unsigned long long u64;

// What a helper learns from its decision record (plain data).  No value of the
// workspace sets the top ("fresh") bit of its 64-bit word: 32-bit values sit in
// the low half, and the chunk statistics keep their never-negative sum or
// argmax in the high half below that bit, so only a hand-off word in flight
// has it set.
struct Setup {
  double Sp, Sq;
  float Mp, Mq;
  int a;
};

struct Params {
  const void* target;
  const void* draft;
  const int32_t* kind;
  const int32_t* cu;
  const int32_t* drafts;
  const float* u;
  const float* temp;
  const int32_t* top_k;
  const float* top_p;
  int32_t* accepted;
  int32_t* out;
  float* p_at;
  float* q_at;
  int32_t* status;
  u64* cst;       // [rows][nc]     target chunk statistics: max in the low half, sum or
                  //                argmax in the high half below the tag (never negative)
  u64* dst;       // [draft rows][nc]
  u64* rx;        // [rows][3]      values at the draft id: l_x, e_x, draft l_x or q(x)
  u64* dec;       // [batch][nc][DEC_W] helper decision records
  u64* res;       // [batch][nc][nc] residual masses sent between helpers ([batch][nc] for nc > PEER_MAX)
  u64* thr_t;     // NULL when no request filters; float bits in the low half
  u64* thr_d;
  u64* pq;        // [batch][2 * max_k] p(x_i), q(x_i) handed to the last helper of a request
  u64* ctl;       // [0]: nonzero once a wait ran out (the workspace is poisoned)
  // penalties (the penalized entry point; pen == nullptr otherwise): the
  // target rows of a request with a nonzero penalty are read from pen, a
  // copy with the same pitch in which k_penalize has penalized them
  const void* pen;
  const float* pres;
  const float* freq;
  const int32_t* hist_off;   // [batch + 1] CSR offsets of the generated-token counts
  const int32_t* hist_tok;   // [hist_nnz] token ids
  const int32_t* hist_cnt;   // [hist_nnz] counts
  int64_t hist_nnz;
  int64_t ld_t, ld_d;
  int batch, total_rows, max_k, vocab, nc;
  int S;          // chunks per producer strip
  int ns;         // strips per row
  int H;          // helper workgroups per request (nc, or 0 for the greedy entry)
  int greedy_entry;
  int dsplit;     // draft-logit rows are read by draft strips of their own
  // batches of more than 64 requests (the kernels instantiated with E = 16):
  // k_order's table of the requests in launch order (request, cu0, cu1,
  // class | valid << 2) and each request's offsets verdict; smaller batches
  // look requests up in place
  int32_t* order;   // [batch][4]
  int32_t* okb;
};

// ---------------------------------------------------------------------------
// element access
// ---------------------------------------------------------------------------
template <typename T> struct VT;
template <> struct VT<float> { static constexpr int VEC = 4; };
template <> struct VT<uint16_t> { static constexpr int VEC = 8; };

__device__ __forceinline__ float to_f(float x) { return x; }
__device__ __forceinline__ float to_f(uint16_t x) { return __uint_as_float((uint32_t)x << 16); }

__device__ __forceinline__ float fmax3nan(float a, float b) {
  return __builtin_elementwise_maximum(a, b);   // NaN-propagating
}

// A thread's share of one chunk, kept as the raw 128-bit words it was loaded
// in (EPT elements); elements are unpacked when they are used.
template <typename T>
struct Seg {
  static constexpr int VEC = VT<T>::VEC;
  static constexpr int NV = EPT / VEC;
  uint4 q[NV];
  __device__ __forceinline__ float at(int i) const;
};
__device__ __forceinline__ uint32_t word_of(const uint4& w, int h) {
  return h == 0 ? w.x : h == 1 ? w.y : h == 2 ? w.z : w.w;
}
template <> __device__ __forceinline__ float Seg<float>::at(int i) const {
  return __uint_as_float(word_of(q[i / 4], i % 4));
}
template <> __device__ __forceinline__ float Seg<uint16_t>::at(int i) const {
  const uint32_t u = word_of(q[i / 8], (i % 8) / 2);
  return __uint_as_float((i & 1) ? (u & 0xffff0000u) : (u << 16));
}

// Element i (0 <= i < EPT, any lane-dependent value) of a thread's words kept in
// LDS, in the layout of Seg::at.
template <typename T> __device__ __forceinline__ float elem_at(const uint4* q, int i);
template <> __device__ __forceinline__ float elem_at<float>(const uint4* q, int i) {
  return __uint_as_float(reinterpret_cast<const uint32_t*>(q)[i]);
}
template <> __device__ __forceinline__ float elem_at<uint16_t>(const uint4* q, int i) {
  return to_f(reinterpret_cast<const uint16_t*>(q)[i]);
}

// 32-bit pattern of `fill` in the element type (bf16: the upper half of f32)
template <typename T> __device__ __forceinline__ uint32_t fill_bits(float f);
template <> __device__ __forceinline__ uint32_t fill_bits<float>(float f) { return __float_as_uint(f); }
template <> __device__ __forceinline__ uint32_t fill_bits<uint16_t>(float f) { return __float_as_uint(f) >> 16; }

__device__ __forceinline__ uint32_t raw_bits(float x) { return __float_as_uint(x); }
__device__ __forceinline__ uint32_t raw_bits(uint16_t x) { return (uint32_t)x; }

// Elements [nv, VEC) of a loaded word replaced by the fill pattern.
template <typename T>
__device__ __forceinline__ uint4 mask_tail(uint4 w, int nv, uint32_t fb) {
  constexpr int VEC = VT<T>::VEC;
  uint32_t d[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    if (VEC == 4) {
      d[k] = (k < nv) ? d[k] : fb;
    } else {
      const uint32_t lo = (2 * k < nv) ? (d[k] & 0xffffu) : fb;
      const uint32_t hi = (2 * k + 1 < nv) ? (d[k] >> 16) : fb;
      d[k] = lo | (hi << 16);
    }
  }
  return make_uint4(d[0], d[1], d[2], d[3]);
}

// One 128-bit word of elements [off, off + VEC) of the chunk at cp, element
// loads with `fill` from element n on (tensors whose rows are not 16-byte
// aligned).
template <typename T>
__device__ __forceinline__ uint4 load_word_scalar(const T* __restrict__ cp, int off, int n,
                                                  float fill) {
  constexpr int VEC = VT<T>::VEC;
  const uint32_t fb = fill_bits<T>(fill);
  uint32_t e[VEC];
#pragma unroll
  for (int l = 0; l < VEC; ++l) e[l] = (off + l < n) ? raw_bits(cp[off + l]) : fb;
  uint4 w;
  if (VEC == 4) {
    w.x = e[0]; w.y = e[1]; w.z = e[2]; w.w = e[3];
  } else {
    w.x = e[0] | (e[1 % VEC] << 16); w.y = e[2 % VEC] | (e[3 % VEC] << 16);
    w.z = e[4 % VEC] | (e[5 % VEC] << 16); w.w = e[6 % VEC] | (e[7 % VEC] << 16);
  }
  return w;
}

// Fill the thread's words, word i at element offset offs(i) of the chunk at cp
// (n valid elements).  al: the tensor's base address and row pitch are
// multiples of 16 bytes, so every word is one 128-bit load issued from an
// offset clamped to the last word that starts inside the row (always inside the
// row's pitch); finish_words then masks the tail past n.  issue_words returns
// without waiting for the data, so a chunk's loads can be in flight while the
// previous chunk is reduced.
// One 128-bit word loaded without keeping it in the caches (rows the producers
// read once).
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ld_stream(const void* p) {
  const u32x4 t = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(t.x, t.y, t.z, t.w);
}

template <typename T, typename OF, bool NT = false>
__device__ __forceinline__ void issue_words(const T* __restrict__ cp, int n, bool al, float fill,
                                            OF offs, Seg<T>& s) {
  constexpr int VEC = VT<T>::VEC;
  if (al) {
    const int last = ((n - 1) / VEC) * VEC;
#pragma unroll
    for (int i = 0; i < Seg<T>::NV; ++i)
      s.q[i] = NT ? ld_stream(cp + min(offs(i), last))
                  : *reinterpret_cast<const uint4*>(cp + min(offs(i), last));
  } else {
#pragma unroll
    for (int i = 0; i < Seg<T>::NV; ++i) s.q[i] = load_word_scalar<T>(cp, offs(i), n, fill);
  }
}

template <typename T, typename OF>
__device__ __forceinline__ void finish_words(int n, bool al, float fill, OF offs, Seg<T>& s) {
  if (al && n < CHUNK) {   // uniform: only the last chunk of a row is partial
    const uint32_t fb = fill_bits<T>(fill);
#pragma unroll
    for (int i = 0; i < Seg<T>::NV; ++i) s.q[i] = mask_tail<T>(s.q[i], n - offs(i), fb);
  }
}

template <typename T, typename OF>
__device__ __forceinline__ void load_words(const T* __restrict__ cp, int n, bool al, float fill,
                                           OF offs, Seg<T>& s) {
  issue_words<T>(cp, n, al, fill, offs, s);
  finish_words<T>(n, al, fill, offs, s);
}

template <typename T>
__device__ __forceinline__ int strided_off(int i) {
  return (i * WG + (int)threadIdx.x) * VT<T>::VEC;
}

// element index in the chunk of the thread's slot (word slot / VEC, lane slot % VEC)
template <typename T>
__device__ __forceinline__ int strided_index(int slot) {
  constexpr int VEC = VT<T>::VEC;
  return strided_off<T>(slot / VEC) + slot % VEC;
}

// Contiguous layout: thread tid holds elements [tid*EPT, tid*EPT + EPT) in
// token order (used by the final draws, which scan in token order).
template <typename T>
__device__ __forceinline__ void load_contig(const T* __restrict__ cp, int n, bool al, float fill,
                                            Seg<T>& s) {
  constexpr int VEC = VT<T>::VEC;
  if (al && n >= CHUNK) {
    // a whole chunk (uniform): one base address, the words at immediate
    // offsets, nothing to clamp or mask
    const uint4* base = reinterpret_cast<const uint4*>(cp + (int)threadIdx.x * EPT);
#pragma unroll
    for (int i = 0; i < Seg<T>::NV; ++i) s.q[i] = base[i];
    return;
  }
  load_words<T>(cp, n, al, fill, [](int i) { return (int)threadIdx.x * EPT + i * VEC; }, s);
}

// ---------------------------------------------------------------------------
// hand-off words (see the file comment)
// ---------------------------------------------------------------------------
template <typename T>
__device__ __forceinline__ void st_agent(T* p, T v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <typename T>
__device__ __forceinline__ T ld_agent(const T* p) {
  return __hip_atomic_load(const_cast<T*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void put_w(u64* w, uint32_t flags, uint32_t payload) {
  st_agent(w, ((u64)(TAG | flags) << 32) | (u64)payload);
}
__device__ __forceinline__ uint32_t hi32(u64 v) { return (uint32_t)(v >> 32); }
__device__ __forceinline__ uint32_t lo32(u64 v) { return (uint32_t)v; }

// Wait for the tag of *w, consume the word (store it back untagged, payload
// kept) and return it; returns 0 (no tag) when the wait runs out.
__device__ __forceinline__ u64 take_w(u64* w) {
  for (int it = 0; it < SPIN_MAX; ++it) {
    const u64 v = ld_agent(w);
    if (hi32(v) & TAG) {
      st_agent(w, v & ((u64)(~TAG) << 32 | 0xffffffffull));
      return v;
    }
    __builtin_amdgcn_s_sleep(1);
  }
  return 0ull;
}

// A wait that ran out leaves hand-off words in flight that a later call would
// take as fresh: the workspace is marked, and every call on it reports
// SV_ROW_INTERNAL until spec_verify_workspace_init clears the mark.
__device__ __forceinline__ void poison(u64* ctl) { st_agent(ctl, 1ull); }


// ---------------------------------------------------------------------------
// block reductions (fixed order: deterministic)
// ---------------------------------------------------------------------------
struct Smem {
  float f[NWAVE];
  double d[NWAVE];
  int i[NWAVE];
  unsigned long long u[NWAVE];
};

// A read-only input at an address that is the same in every lane, loaded
// through the scalar cache: its wait counter is not the one of the vector
// loads, so waiting for it never waits for the row data in flight.
template <typename T>
__device__ __forceinline__ T ldu(const T* p) {
  return *(const __attribute__((address_space(4))) T*)p;
}

// ---------------------------------------------------------------------------
// per-request parameters
// ---------------------------------------------------------------------------
struct Req {
  float T;
  bool greedy;
  int kind;
  bool bad_param;
  int K;
  float P;
  bool filt;
  float c;    // log2(e) / T rounded to fp32
  double ce;  // the same value in fp64
  bool pen;   // nonzero penalties: the target rows come from the penalized copy
};

// Whether request b has nonzero penalties (only the penalized entry point
// passes them).
__device__ __forceinline__ bool pen_of(const Params& P, int b) {
  return P.pen != nullptr && (ldu(P.pres + b) != 0.f || ldu(P.freq + b) != 0.f);
}
template <typename TT>
__device__ __forceinline__ const TT* target_rows(const Params& P, bool pen) {
  return (const TT*)(pen ? P.pen : P.target);
}

__device__ __forceinline__ Req load_req(const Params& P, int b) {
  Req R;
  // every load goes out at once (their conditions are kernel arguments only);
  // the greedy test then selects what is kept
  const float T = P.greedy_entry ? 0.f : ldu(P.temp + b);
  const int kind = P.greedy_entry ? -1 : ldu(P.kind + b);
  const int K = P.top_k ? ldu(P.top_k + b) : 0;
  const float Pp = P.top_p ? ldu(P.top_p + b) : 1.f;
  R.T = T;
  R.greedy = P.greedy_entry || !(R.T >= FLT_MIN);
  R.kind = R.greedy ? -1 : kind;
  const float ap = P.pen ? ldu(P.pres + b) : 0.f;
  const float af = P.pen ? ldu(P.freq + b) : 0.f;
  R.pen = ap != 0.f || af != 0.f;
  const bool pen_bad = R.pen && !(__builtin_isfinite(ap) && __builtin_isfinite(af));
  R.bad_param = pen_bad ||
                (!R.greedy &&
                 (R.T == POS_INF || R.kind < SV_DRAFT_ONEHOT || R.kind > SV_DRAFT_MATCH ||
                  ((R.kind == SV_DRAFT_LOGITS || R.kind == SV_DRAFT_PROBS) && P.draft == nullptr)));
  R.K = R.greedy ? 0 : K;
  R.P = R.greedy ? 1.f : Pp;
  if (R.K >= P.vocab) R.K = 0;
  R.filt = R.K > 0 || (R.P > 0.f && R.P < 1.f);
  if (!R.greedy && !R.bad_param) {
    R.c = (float)(LOG2E / (double)R.T);   // finite and > 0 for FLT_MIN <= T < inf
    R.ce = (double)R.c;
  } else {
    R.c = 0.f;
    R.ce = 0.0;
  }
  return R;
}

__device__ __forceinline__ bool req_valid(const Params& P, int b, int cu0, int cu1, int k) {
  return cu0 >= 0 && cu1 <= P.total_rows && k >= 0 && k <= P.max_k && cu0 - b >= 0 &&
         cu0 - b + k <= P.total_rows - P.batch;
}

__device__ __forceinline__ float thr_of(const u64* t, int i) {
  return __uint_as_float((uint32_t)ldu(t + i));
}

// exp2((v - r) * c) for v <= r, r finite (v = -inf gives 0)
__device__ __forceinline__ float term(float v, float r, float c) {
  return __builtin_amdgcn_exp2f((v - r) * c);
}

// exp2(v * c - mc) with one rounding of the argument (v = -inf gives 0)
__device__ __forceinline__ float fterm(float v, float c, float mc) {
  return __builtin_amdgcn_exp2f(__builtin_fmaf(v, c, -mc));
}

// exp2((m - M) * c) in fp64 (the scale of a chunk with max m in a row with max M)
__device__ __forceinline__ double scale_d(float m, float M, double ce) {
  return exp2(((double)m - (double)M) * ce);
}

// ---------------------------------------------------------------------------
// producers: statistics of one chunk of one row
// ---------------------------------------------------------------------------
struct CStat {
  float m;     // chunk max (NaN / +inf propagate)
  float s;     // sum of element terms relative to m (sampled rows)
  float sx;    // the same sum without the element xl (when asked for)
  int arg;     // lowest index of the max within the chunk (greedy rows)
};

// ---- wave reductions over DPP: rows of 16 lanes by butterflies, then the four
// rows read back as scalars (the result is uniform across the wave)
template <int CTRL>
__device__ __forceinline__ int dpp_i(int x) {
  return __builtin_amdgcn_update_dpp(x, x, CTRL, 0xf, 0xf, false);
}
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
  return __int_as_float(dpp_i<CTRL>(__float_as_int(x)));
}
template <int CTRL>
__device__ __forceinline__ double dpp_d(double x) {
  const long long v = __double_as_longlong(x);
  const int lo = dpp_i<CTRL>((int)(uint32_t)v);
  const int hi = dpp_i<CTRL>((int)(uint32_t)(v >> 32));
  return __longlong_as_double((long long)(((u64)(uint32_t)hi << 32) | (u64)(uint32_t)lo));
}
// x from the lane CTRL names, +0.0 where the control names no lane (bound off)
template <int CTRL, int ROWS>
__device__ __forceinline__ double dpp_or0_d(double x) {
  const long long v = __double_as_longlong(x);
  const int lo = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)v, CTRL, ROWS, 0xf, false);
  const int hi = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)(v >> 32), CTRL, ROWS, 0xf, false);
  return __longlong_as_double((long long)(((u64)(uint32_t)hi << 32) | (u64)(uint32_t)lo));
}
static_assert(EPT == 32, "the draw's segment scan covers 32 lanes");
// Inclusive fp64 scan over the wave: row shifts of 1, 2, 4, 8, then the last
// value of rows 0 and 2 into rows 1 and 3, then lane 31 into rows 2 and 3.
__device__ __forceinline__ double scan64_d(double x) {
  x += dpp_or0_d<0x111, 0xf>(x);   // row_shr:1
  x += dpp_or0_d<0x112, 0xf>(x);   // row_shr:2
  x += dpp_or0_d<0x114, 0xf>(x);   // row_shr:4
  x += dpp_or0_d<0x118, 0xf>(x);   // row_shr:8
  x += dpp_or0_d<0x142, 0xa>(x);   // row_bcast:15 into rows 1 and 3
  x += dpp_or0_d<0x143, 0xc>(x);   // row_bcast:31 into rows 2 and 3
  return x;
}
// Inclusive fp64 scan over lanes 0..31 (row shifts of 1, 2, 4, 8, then row 0's
// last value into row 1); lanes 32..63 hold their own partial values.
__device__ __forceinline__ double scan32_d(double x) {
  x += dpp_or0_d<0x111, 0xf>(x);   // row_shr:1
  x += dpp_or0_d<0x112, 0xf>(x);   // row_shr:2
  x += dpp_or0_d<0x114, 0xf>(x);   // row_shr:4
  x += dpp_or0_d<0x118, 0xf>(x);   // row_shr:8
  x += dpp_or0_d<0x142, 0x2>(x);   // row_bcast:15 into row 1
  return x;
}

constexpr int DPP_XOR1 = 0xB1;      // quad_perm [1,0,3,2]
constexpr int DPP_XOR2 = 0x4E;      // quad_perm [2,3,0,1]
constexpr int DPP_HMIRROR = 0x141;  // lane i <-> 7 - i within each 8
constexpr int DPP_MIRROR = 0x140;   // lane i <-> 15 - i within each 16

__device__ __forceinline__ float rl_f(float x, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), l));
}
__device__ __forceinline__ double rl_d(double x, int l) {
  const long long v = __double_as_longlong(x);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, l);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), l);
  return __longlong_as_double((long long)(((u64)hi << 32) | lo));
}

template <int CTRL> __device__ __forceinline__ float dpp_any(float x) { return dpp_f<CTRL>(x); }
template <int CTRL> __device__ __forceinline__ int dpp_any(int x) { return dpp_i<CTRL>(x); }
template <int CTRL> __device__ __forceinline__ double dpp_any(double x) { return dpp_d<CTRL>(x); }
__device__ __forceinline__ float rl_any(float x, int l) { return rl_f(x, l); }
__device__ __forceinline__ int rl_any(int x, int l) { return __builtin_amdgcn_readlane(x, l); }
__device__ __forceinline__ double rl_any(double x, int l) { return rl_d(x, l); }

// Block reductions: DPP within each 16-lane row, the four rows of a wave read
// from lanes 0, 16, 32, 48, the waves through LDS in wave order.
template <typename T, typename OP>
__device__ __forceinline__ T wave_reduce_rows(T x, OP op) {
  x = op(x, dpp_any<DPP_XOR1>(x));
  x = op(x, dpp_any<DPP_XOR2>(x));
  x = op(x, dpp_any<DPP_HMIRROR>(x));
  x = op(x, dpp_any<DPP_MIRROR>(x));
  return op(op(rl_any(x, 0), rl_any(x, 16)), op(rl_any(x, 32), rl_any(x, 48)));
}

__device__ __forceinline__ float block_max(float x, Smem& sm) {
  x = wave_reduce_rows(x, [](float a, float b) { return fmax3nan(a, b); });
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) sm.f[w] = x;
  __syncthreads();
  float r = sm.f[0];
#pragma unroll
  for (int k = 1; k < NWAVE; ++k) r = fmax3nan(r, sm.f[k]);
  return r;
}

__device__ __forceinline__ int block_max_i(int x, Smem& sm) {
  x = wave_reduce_rows(x, [](int a, int b) { return max(a, b); });
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) sm.i[w] = x;
  __syncthreads();
  int r = sm.i[0];
#pragma unroll
  for (int k = 1; k < NWAVE; ++k) r = max(r, sm.i[k]);
  return r;
}

__device__ __forceinline__ double block_sum_d(double x, Smem& sm) {
  x = wave_reduce_rows(x, [](double a, double b) { return a + b; });
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) sm.d[w] = x;
  __syncthreads();
  double r = sm.d[0];
#pragma unroll
  for (int k = 1; k < NWAVE; ++k) r += sm.d[k];
  return r;
}

// Inclusive fp64 scan over the block in thread order; also returns the
// exclusive value (the inclusive value of the previous thread).
__device__ __forceinline__ void block_scan_d(double own, double& excl, double& incl, Smem& sm) {
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  double x = scan64_d(own);   // within the wave (DPP)
  __syncthreads();
  if (lane == 63) sm.d[w] = x;
  __syncthreads();
  double carry = 0.0;
  for (int k = 0; k < w; ++k) carry += sm.d[k];
  x += carry;
  const double prev = dpp_or0_d<0x138, 0xf>(x);   // wave_shr:1
  incl = x;
  excl = (lane == 0) ? carry : prev;
}

// The same scan, also returning the block total (the inclusive value of the
// last thread, summed in the same order).
__device__ __forceinline__ void block_scan_total_d(double own, double& excl, double& incl,
                                                   double& total, Smem& sm) {
  block_scan_d(own, excl, incl, sm);
  double t = sm.d[0];
#pragma unroll
  for (int k = 1; k < NWAVE; ++k) t += sm.d[k];
  total = t;
}


__device__ __forceinline__ float wave_max(float x) {
  x = fmax3nan(x, dpp_f<DPP_XOR1>(x));
  x = fmax3nan(x, dpp_f<DPP_XOR2>(x));
  x = fmax3nan(x, dpp_f<DPP_HMIRROR>(x));
  x = fmax3nan(x, dpp_f<DPP_MIRROR>(x));
  return fmax3nan(fmax3nan(rl_f(x, 0), rl_f(x, 16)), fmax3nan(rl_f(x, 32), rl_f(x, 48)));
}

// Sum in a fixed tree order (lane pairs, quads, halves, rows, then rows 0..3).
__device__ __forceinline__ double wave_sum(double x) {
  x += dpp_d<DPP_XOR1>(x);
  x += dpp_d<DPP_XOR2>(x);
  x += dpp_d<DPP_HMIRROR>(x);
  x += dpp_d<DPP_MIRROR>(x);
  return (rl_d(x, 0) + rl_d(x, 16)) + (rl_d(x, 32) + rl_d(x, 48));
}

// (max, lowest index of the max); NaN propagates with index INT32_MAX
__device__ __forceinline__ void arg_step(float& m, int& i, float mo, int io) {
  const float mm = fmax3nan(m, mo);
  i = min(m == mm ? i : INT32_MAX, mo == mm ? io : INT32_MAX);
  m = mm;
}
template <int CTRL>
__device__ __forceinline__ void arg_dpp(float& m, int& i) {
  arg_step(m, i, dpp_f<CTRL>(m), dpp_i<CTRL>(i));
}
__device__ __forceinline__ void wave_argmax(float& m, int& i) {
  arg_dpp<DPP_XOR1>(m, i);
  arg_dpp<DPP_XOR2>(m, i);
  arg_dpp<DPP_HMIRROR>(m, i);
  arg_dpp<DPP_MIRROR>(m, i);
  float m0 = rl_f(m, 0);
  int i0 = __builtin_amdgcn_readlane(i, 0);
#pragma unroll
  for (int r = 16; r < 64; r += 16) arg_step(m0, i0, rl_f(m, r), __builtin_amdgcn_readlane(i, r));
  m = m0;
  i = i0;
}

// LDS of the producer reductions: two slot sets used alternately by
// consecutive chunks, so each reduction needs a single barrier.
struct ProdShared {
  float m[2][NWAVE];
  int i[2][NWAVE];
  double s[2][NWAVE];
  double sx[2][NWAVE];
  uint32_t pub[16][3];   // per task: max, sum or index, sum without x
};

// Mask, in place, every element below tau (a top-k / top-p threshold) to -inf.
// NaN compares false and is kept, so the fault is still seen.
__device__ __forceinline__ uint32_t mask16(uint32_t h, float tau) {
  return (__uint_as_float(h << 16) < tau) ? 0xff80u : h;
}
template <typename T> __device__ __forceinline__ void apply_tau(Seg<T>& sg, float tau);
template <> __device__ __forceinline__ void apply_tau<float>(Seg<float>& sg, float tau) {
#pragma unroll
  for (int i = 0; i < Seg<float>::NV; ++i) {
    uint32_t d[4] = {sg.q[i].x, sg.q[i].y, sg.q[i].z, sg.q[i].w};
#pragma unroll
    for (int k = 0; k < 4; ++k) d[k] = (__uint_as_float(d[k]) < tau) ? 0xff800000u : d[k];
    sg.q[i] = make_uint4(d[0], d[1], d[2], d[3]);
  }
}
template <> __device__ __forceinline__ void apply_tau<uint16_t>(Seg<uint16_t>& sg, float tau) {
#pragma unroll
  for (int i = 0; i < Seg<uint16_t>::NV; ++i) {
    uint32_t d[4] = {sg.q[i].x, sg.q[i].y, sg.q[i].z, sg.q[i].w};
#pragma unroll
    for (int k = 0; k < 4; ++k) d[k] = mask16(d[k] & 0xffffu, tau) | (mask16(d[k] >> 16, tau) << 16);
    sg.q[i] = make_uint4(d[0], d[1], d[2], d[3]);
  }
}


// Statistics of one chunk held in the strided layout (slot i of the thread is
// chunk element strided_index(i)).  xl: chunk-local index of the draft id, or
// -1.  par: the slot set of this chunk.  All threads return the same values.
template <typename T>
__device__ __forceinline__ CStat chunk_stats(Seg<T>& sg, bool greedy, float tau, float c, int xl,
                                             int par, ProdShared& ps, bool before = false) {
  if (tau > NEG_INF) apply_tau<T>(sg, tau);
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  float m = NEG_INF;
#pragma unroll
  for (int i = 0; i < EPT; ++i) m = fmax3nan(m, sg.at(i));
  CStat st;
  st.s = 0.f;
  st.sx = 0.f;
  st.arg = INT32_MAX;
  if (greedy) {
    int slot = EPT;
#pragma unroll
    for (int i = EPT - 1; i >= 0; --i) slot = (sg.at(i) == m) ? i : slot;
    float wm = m;
    int wi = slot < EPT ? strided_index<T>(slot) : INT32_MAX;
    wave_argmax(wm, wi);
    if (lane == 0) {
      ps.m[par][w] = wm;
      ps.i[par][w] = wi;
    }
    __syncthreads();
    float bm = ps.m[par][0];
    int bi = ps.i[par][0];
#pragma unroll
    for (int q = 1; q < NWAVE; ++q) arg_step(bm, bi, ps.m[par][q], ps.i[par][q]);
    st.m = bm;
    st.arg = bi;
    return st;
  }
  const float wm = wave_max(m);
  if (lane == 0) ps.m[par][w] = wm;
  // the terms against the thread's own max need no block result: they run
  // while the other waves reach the barrier.  Each term is exp2(l*c - mc) with
  // mc = m*c rounded once and the argument rounded once (one fused
  // multiply-add); the common factor exp2(m*c - mc) is put back exactly when the
  // thread's sum is scaled to the chunk max below.
  // The rounding error of mc enters every term as a factor exp2(err) that the
  // scale below takes out again; it stays harmless while |mc| < 2^30 (|err| <
  // 64).  Beyond that (a huge |m|, or a tiny temperature) the thread takes the
  // terms exp2((l - m) * c) instead, which cannot overflow for l <= m, and
  // scales them to the chunk max by exp2((m - M) * c).  The one-FMA loops
  // always run (a per-thread choice between two loops slowed the common
  // case); a wave that holds such a thread redoes it afterwards, on a
  // wave-uniform branch.
  float acc = 0.f, accx = 0.f;
  const bool own = m > NEG_INF && m < POS_INF;
  const float mc = m * c;
  const bool fast = __builtin_fabsf(mc) < 1073741824.0f;
  constexpr int VEC = VT<T>::VEC;
  const int owner = xl >= 0 ? (xl / VEC) % WG : -1;
  const int xslot = xl >= 0 ? ((xl / VEC) / WG) * VEC + xl % VEC : -1;
  const int ix = ((int)threadIdx.x == owner) ? xslot : -1;
  if (xl < 0) {
    if (own) {
#pragma unroll
      for (int i = 0; i < EPT; ++i) acc += fterm(sg.at(i), c, mc);
    }
  } else if (own) {
    if (before) {
      // the terms of the elements that precede x in token order
#pragma unroll
      for (int i = 0; i < EPT; ++i) {
        const float e = fterm(sg.at(i), c, mc);
        acc += e;
        accx += (strided_index<T>(i) < xl) ? e : 0.f;
      }
    } else {
#pragma unroll
      for (int i = 0; i < EPT; ++i) {
        const float e = fterm(sg.at(i), c, mc);
        acc += e;
        accx += (i == ix) ? 0.f : e;
      }
    }
  }
  if (__ballot(own && !fast)) {
    if (own && !fast) {
      acc = 0.f;
      accx = 0.f;
#pragma unroll
      for (int i = 0; i < EPT; ++i) {
        // a rare path: each value passes an empty asm statement with the
        // running sums, so its term is formed after the previous one is
        // added instead of every term being held at once
        float v = sg.at(i);
        asm volatile("" : "+v"(v), "+v"(acc), "+v"(accx));
        const float e = term(v, m, c);
        acc += e;
        accx += (xl < 0) ? 0.f
                : before ? ((strided_index<T>(i) < xl) ? e : 0.f)
                         : ((i == ix) ? 0.f : e);
      }
    }
  }
  __syncthreads();
  float M = ps.m[par][0];
#pragma unroll
  for (int q = 1; q < NWAVE; ++q) M = fmax3nan(M, ps.m[par][q]);
  st.m = M;
  if (!(M > NEG_INF && M < POS_INF)) return st;   // empty chunk or a data fault
  const double f = !own ? 0.0 : fast ? (double)fterm(-M, c, -mc)   // exp2(mc - M*c)
                                     : (double)term(m, M, c);
  const double ws = wave_sum((double)acc * f);
  double wsx = 0.0;
  if (xl >= 0) wsx = wave_sum((double)accx * f);
  if (lane == 0) {
    ps.s[par][w] = ws;
    ps.sx[par][w] = wsx;
  }
  __syncthreads();
  double S = 0.0, SX = 0.0;
#pragma unroll
  for (int q = 0; q < NWAVE; ++q) {
    S += ps.s[par][q];
    SX += ps.sx[par][q];
  }
  st.s = (float)S;
  st.sx = (float)SX;
  return st;
}

// chunks per producer strip (64 KiB of bf16 or fp32 target data)
template <typename TT> struct Strip;
#ifndef SV_STRIP_BF16
#define SV_STRIP_BF16 4
#endif
template <> struct Strip<uint16_t> { static constexpr int S = SV_STRIP_BF16; };
template <> struct Strip<float> { static constexpr int S = (SV_STRIP_BF16 + 1) / 2; };
static_assert(Strip<uint16_t>::S <= 8 && Strip<float>::S <= 8, "strip too long");

// Words of one chunk of either element type (sized for the wider one).
template <typename TT, typename TD>
struct Buf {
  static constexpr int NQ = Seg<TT>::NV > Seg<TD>::NV ? Seg<TT>::NV : Seg<TD>::NV;
  uint4 q[NQ];
};

template <typename T, typename TT, typename TD>
__device__ __forceinline__ void buf_issue(const T* __restrict__ cp, int n, bool al,
                                          Buf<TT, TD>& b) {
  Seg<T> sg;
  auto offs = [](int i) { return strided_off<T>(i); };
  issue_words<T, decltype(offs), true>(cp, n, al, NEG_INF, offs, sg);
#pragma unroll
  for (int i = 0; i < Seg<T>::NV; ++i) b.q[i] = sg.q[i];
}

template <typename TT, typename TD, bool AL>
__device__ __forceinline__ void issue_task(const TT* trow, const TD* drow, bool is_d, int c,
                                           int vocab, Buf<TT, TD>& bf) {
  const int n = min(CHUNK, vocab - c * CHUNK);
  if (is_d) buf_issue<TD>(drow + c * CHUNK, n, AL, bf);
  else buf_issue<TT>(trow + c * CHUNK, n, AL, bf);
}

// One producer task: the statistics of chunk c of the target row (is_d false)
// or of the draft-logit row, kept in LDS (slot t) until the strip ends.  For
// the chunk holding the draft id x, the sum of the terms without x (or, for a
// prefix-match request, of the terms before x) is kept as well.
template <typename T, typename TT, typename TD, bool AL>
__device__ __forceinline__ void produce_task(const Params& P, const Req& R, const Buf<TT, TD>& bf,
                                             bool is_d, int c, int x, float tau, int t,
                                             ProdShared& ps) {
  const int c0 = c * CHUNK;
  const int n = min(CHUNK, P.vocab - c0);
  const bool xin = !is_d && x >= c0 && x < c0 + n;
  Seg<T> sg;
#pragma unroll
  for (int i = 0; i < Seg<T>::NV; ++i) sg.q[i] = bf.q[i];
  finish_words<T>(n, AL, NEG_INF, [](int i) { return strided_off<T>(i); }, sg);
  const bool greedy = R.greedy && !is_d;
  const CStat st = chunk_stats<T>(sg, greedy, tau, R.c, xin ? x - c0 : -1, t & 1, ps,
                                  R.kind == SV_DRAFT_MATCH);
  if (threadIdx.x == 0) {
    ps.pub[t][0] = __float_as_uint(st.m);
    ps.pub[t][1] = greedy ? (uint32_t)st.arg : __float_as_uint(st.s);
    ps.pub[t][2] = __float_as_uint(st.sx);
  }
}

// Producer of request b, target row j, strip s: statistics of S chunks of the
// target row, and the single values at the draft id when it falls in the
// strip.  Draft rows are read by draft strips of their own (produce_draft).
// The hand-off words are written after the strip.
template <typename TT, typename TD, bool AL>
__device__ __forceinline__ void produce(const Params& P, const Req& R, int b, int cu0, int k,
                                        int j, int s, ProdShared& ps, Buf<TT, TD>& A) {
  const int nc = P.nc;
  const int row = cu0 + j;
  const int d0 = cu0 - b;
  const TT* trow = target_rows<TT>(P, R.pen) + (int64_t)row * P.ld_t;
  // the draft id and the thresholds are loaded without waiting for the
  // request's parameters, which only decide whether they are used
  const int xr = j < k ? ldu(P.drafts + d0 + j) : -1;
  const float tau_r = P.thr_t ? thr_of(P.thr_t, row) : NEG_INF;
  const float tau = R.filt ? tau_r : NEG_INF;
  const TD* drow = (const TD*)P.draft + (int64_t)(d0 + j) * P.ld_d;
  const int x = R.greedy ? -1 : xr;
  const int c_begin = s * P.S;
  const int c_end = min(c_begin + P.S, nc);
  const int nt = c_end - c_begin;
  // the single values at the draft id, gathered by thread 0 and published
  // after the strip (issued first, they wait behind nothing)
  const bool xs = threadIdx.x == 0 && x >= c_begin * CHUNK && x < min(c_end * CHUNK, P.vocab);
  TT lx_raw = TT(0);
  TD ldx_raw = TD(0);
  if (xs) {
    lx_raw = trow[x];
    if (R.kind == SV_DRAFT_LOGITS || R.kind == SV_DRAFT_PROBS) ldx_raw = drow[x];
  }

  // two chunks in flight: chunk t+1 is requested before chunk t is reduced.
  // Past the row's last chunk the loads repeat it (never reduced).  Two
  // chunks per workgroup keep the memory busy with every slot of the GPU
  // filled, and fewer bytes queued ahead of every load shorten the dependent
  // round trips that follow the statistics.
  constexpr int S = Strip<TT>::S;
  Buf<TT, TD> Q[S];
  Q[0] = A;
#pragma unroll
  for (int t = 0; t < S; ++t) {
    if (t + 1 < S)
      issue_task<TT, TD, AL>(trow, drow, false, c_begin + min(t + 1, nt - 1), P.vocab, Q[t + 1]);
    if (t < nt) produce_task<TT, TT, TD, AL>(P, R, Q[t], false, c_begin + t, x, tau, t, ps);
  }
  __syncthreads();
  const int tp = threadIdx.x;
  if (tp < nt) {
    const int c = c_begin + tp;
    // one word per chunk: the sum (or argmax) is never negative, so its top
    // bit is free for the tag
    put_w(P.cst + ((int64_t)row * nc + c), ps.pub[tp][1] & ~TAG, ps.pub[tp][0]);
    const int c0 = c * CHUNK;
    if (x >= c0 && x < c0 + min(CHUNK, P.vocab - c0))
      put_w(P.rx + (int64_t)row * 3 + 1, 0u, ps.pub[tp][2]);
  }
  if (xs) {
    // the draft value at x goes out raw: a draft logit is masked by the
    // finalizer, which reads the draft row's threshold
    float lx = to_f(lx_raw);
    if (lx < tau) lx = NEG_INF;
    put_w(P.rx + (int64_t)row * 3 + 0, 0u, __float_as_uint(lx));
    if (R.kind == SV_DRAFT_PROBS || R.kind == SV_DRAFT_LOGITS)
      put_w(P.rx + (int64_t)row * 3 + 2, 0u, __float_as_uint(to_f(ldx_raw)));
  }
}

// Draft strip of request b, draft row j, strip s (draft-logit requests): the
// statistics of S chunks of the draft row, three chunks in flight (chunks t+1
// and t+2 are requested before chunk t is reduced), published to the draft
// hand-off words.  Draft strips come first in the grid, so the draft rows
// stream while the target strips start, with the same bytes per workgroup;
// with fewer workgroups streaming beside them than the producers have, a
// deeper window pays here.
template <typename TT, typename TD, bool AL>
__device__ __forceinline__ void produce_draft(const Params& P, const Req& R, int b, int cu0, int j,
                                              int s, ProdShared& ps, Buf<TT, TD>& A) {
  const int nc = P.nc;
  const int d0 = cu0 - b;
  const TD* drow = (const TD*)P.draft + (int64_t)(d0 + j) * P.ld_d;
  const float taud_r = P.thr_d ? thr_of(P.thr_d, d0 + j) : NEG_INF;
  const float taud = R.filt ? taud_r : NEG_INF;
  const int c_begin = s * P.S;
  const int c_end = min(c_begin + P.S, nc);
  const int nt = c_end - c_begin;
  constexpr int S = Strip<TT>::S;
  Buf<TT, TD> Q[S];
  Q[0] = A;
  if (S > 1) issue_task<TT, TD, AL>((const TT*)nullptr, drow, true, c_begin + min(1, nt - 1), P.vocab, Q[1]);
#pragma unroll
  for (int t = 0; t < S; ++t) {
    if (t + 2 < S)
      issue_task<TT, TD, AL>((const TT*)nullptr, drow, true, c_begin + min(t + 2, nt - 1), P.vocab, Q[t + 2]);
    if (t < nt) produce_task<TD, TT, TD, AL>(P, R, Q[t], true, c_begin + t, -1, taud, t, ps);
  }
  __syncthreads();
  const int tp = threadIdx.x;
  if (tp < nt)
    put_w(P.dst + ((int64_t)(d0 + j) * nc + c_begin + tp), ps.pub[tp][1] & ~TAG, ps.pub[tp][0]);
}

// ---------------------------------------------------------------------------
// final draw over one chunk in token order
// ---------------------------------------------------------------------------
struct DrawShared {
  double E[MAX_NC];
  uint4 qa[Seg<float>::NV], qb[Seg<float>::NV];   // the winning thread's words (rows A and B)
  double tl;
  double wexcl;
  int chunk;
  int tok;
  int win;
};

// Inverse CDF inside one chunk [c0, c0+n) of a row, in token order, once the
// block scan of the segment sums is known.  Thread tid owns the segment
// [c0 + tid*EPT, c0 + tid*EPT + EPT) of weight sum own, scanned into
// [excl, incl).  weight(a, b, e) gives the fp64 weight of element e from its
// values a (row A) and b (row B, only when TWO); it is evaluated again, on the
// same inputs, for the one segment that is searched: its words reach wave 0
// through LDS.  Returns the first element whose running sum exceeds tl; when
// rounding leaves no segment holding tl (tl at or past the total), the last
// element of positive weight.
template <typename TA, typename TB, bool TWO, typename WF>
__device__ __forceinline__ int draw_scanned(const Seg<TA>& sa, const Seg<TB>& sb, float bfill,
                                            int c0, int n, double tl, WF weight, double own,
                                            double excl, double incl, Smem& sm, DrawShared& ds) {
  const int tid = threadIdx.x;
  if (tid == 0) ds.win = -1;
  __syncthreads();
  if (excl <= tl && tl < incl) ds.win = tid;   // at most one thread: the intervals are disjoint
  __syncthreads();
  int win = ds.win;
  const bool fallback = win < 0;
  if (fallback) win = block_max_i(own > 0.0 ? tid : -1, sm);
  if (win < 0) return -1;   // no positive weight: never drawn from
  if (tid == win) {
    ds.wexcl = excl;
#pragma unroll
    for (int i = 0; i < Seg<TA>::NV; ++i) ds.qa[i] = sa.q[i];
    if (TWO) {
#pragma unroll
      for (int i = 0; i < Seg<TB>::NV; ++i) ds.qb[i] = sb.q[i];
    }
  }
  __syncthreads();
  if (tid < 64) {
    const int l = tid;
    const int off = win * EPT + l;
    const bool ok = l < EPT && off < n;
    const float a = ok ? elem_at<TA>(ds.qa, l) : NEG_INF;
    const float bv = (ok && TWO) ? elem_at<TB>(ds.qb, l) : bfill;
    const double w = ok ? weight(a, bv, c0 + off) : 0.0;
    const double x = scan32_d(w);   // EPT = 32 elements: lanes 0..31
    const uint64_t hit = fallback ? 0ull : __ballot(w > 0.0 && ds.wexcl + x > tl);
    // no hit: the segment's last element of positive weight
    const uint64_t pos = __ballot(w > 0.0);
    const int lastw = pos ? c0 + win * EPT + 63 - (int)__builtin_clzll(pos) : -1;
    if (l == 0) ds.tok = hit ? c0 + win * EPT + (int)__builtin_ctzll(hit) : lastw;
  }
  __syncthreads();
  return ds.tok;
}

// Weight sum of this thread's segment (its interval in the draw's block scan).
template <typename TA, typename TB, bool TWO, typename WF>
__device__ __forceinline__ double seg_weights(const Seg<TA>& sa, const Seg<TB>& sb, int c0,
                                              WF weight) {
  const int seg = threadIdx.x * EPT;
  // two partial sums (even and odd elements) halve the chain of dependent adds
  double own0 = 0.0, own1 = 0.0;
#pragma unroll
  for (int i = 0; i < EPT; i += 2) {
    own0 += weight(sa.at(i), TWO ? sb.at(i) : 0.f, c0 + seg + i);
    own1 += weight(sa.at(i + 1), TWO ? sb.at(i + 1) : 0.f, c0 + seg + i + 1);
    if ((i & 3) == 2) __builtin_amdgcn_sched_barrier(0);   // bound live fp64 temporaries
  }
  return own0 + own1;
}

// The draw over a chunk whose segment sums are not known yet.
template <typename TA, typename TB, bool TWO, typename WF>
__device__ __forceinline__ int draw_held(const Seg<TA>& sa, const Seg<TB>& sb, float bfill, int c0,
                                         int n, double tl, WF weight, Smem& sm, DrawShared& ds) {
  const double own = seg_weights<TA, TB, TWO>(sa, sb, c0, weight);
  double excl, incl;
  block_scan_d(own, excl, incl, sm);
  return draw_scanned<TA, TB, TWO>(sa, sb, bfill, c0, n, tl, weight, own, excl, incl, sm, ds);
}

// The same, loading the chunk (contiguous layout) first.
template <typename TA, typename TB, bool TWO, typename WF>
__device__ __forceinline__ int draw_chunk(const TA* __restrict__ pa, const TB* __restrict__ pb, bool avec,
                          bool bvec, float bfill, int c0, int n, double tl, WF weight, Smem& sm,
                          DrawShared& ds) {
  Seg<TA> sa;
  Seg<TB> sb;
  load_contig<TA>(pa + c0, n, avec, NEG_INF, sa);
  if (TWO) load_contig<TB>(pb + c0, n, bvec, bfill, sb);
  return draw_held<TA, TB, TWO>(sa, sb, bfill, c0, n, tl, weight, sm, ds);
}

// Pick the chunk holding target = u*W given chunk masses in ds.E[0..nc).
// Returns false when W == 0.  Wave 0 scans the masses in blocks of 64 chunks
// (an fp64 wave scan per block, blocks added in order; W is the last prefix,
// so the prefixes and W round alike); result in ds.chunk and ds.tl (target
// minus the prefix before the chunk; +inf when rounding leaves no chunk past
// the target, which then picks the last chunk of positive mass).
__device__ __forceinline__ bool pick_chunk(int nc, double u, DrawShared& ds) {
  __syncthreads();
  if (threadIdx.x < 64) {
    const int l = threadIdx.x;
    double W = 0.0;
    for (int c0 = 0; c0 < nc; c0 += 64) {
      const double e = (c0 + l < nc) ? ds.E[c0 + l] : 0.0;
      W += rl_d(scan64_d(e), 63);
    }
    int ch = -1;
    double tl = 0.0;
    if (W > 0.0) {
      const double target = u * W;
      double pre = 0.0;
      int last = -1;
      for (int c0 = 0; c0 < nc; c0 += 64) {
        const double e = (c0 + l < nc) ? ds.E[c0 + l] : 0.0;
        const double sc = scan64_d(e);
        const uint64_t pos = __ballot(e > 0.0);
        if (pos) last = c0 + 63 - (int)__builtin_clzll(pos);
        const uint64_t hit = __ballot(e > 0.0 && pre + sc > target);
        if (hit) {
          const int li = (int)__builtin_ctzll(hit);
          ch = c0 + li;
          tl = target - (li == 0 ? pre : pre + rl_d(sc, li - 1));
          break;
        }
        pre += rl_d(sc, 63);
      }
      if (ch < 0) {   // rounding: target at or past the total
        ch = last;
        tl = POS_INF;
      }
    }
    if (l == 0) {
      ds.chunk = ch;
      ds.tl = tl;
    }
  }
  __syncthreads();
  return ds.chunk >= 0;
}


// Draw from p of one target row (bonus draw, one-hot rejection with
// `exclude` = the rejected draft id, zero-residual fallback).  cm(c) gives
// chunk c's max, mass(c, ex) its mass scaled to the row max (ex: leave the
// token `exclude` out of x's chunk) and rc(c) that scale, so mass / rc is in
// units of the chunk's own terms.  Returns the token (all threads).
template <typename TT, bool AL, typename FM, typename FS, typename FR>
__device__ __forceinline__ int draw_target_row(const Params& P, const Req& R, int row, int exclude,
                                               float tau, double u, FM cm, FS mass, FR rc,
                                               Smem& sm, DrawShared& ds) {
  const int nc = P.nc;
  for (int attempt = 0; attempt < 2; ++attempt) {
    for (int c = threadIdx.x; c < nc; c += WG) {
      double e = mass(c, exclude >= 0 && exclude / CHUNK == c);
      if (!(e > 0.0)) e = 0.0;
      ds.E[c] = e;
    }
    if (pick_chunk(nc, u, ds)) break;
    if (exclude < 0) return -1;
    exclude = -1;   // only the rejected token had mass: fall back to p itself
  }
  const int ch = ds.chunk;
  const float m = cm(ch);
  const double tl = ds.tl / rc(ch);
  const int c0 = ch * CHUNK;
  const int n = min(CHUNK, P.vocab - c0);
  const TT* rp = target_rows<TT>(P, R.pen) + (int64_t)row * P.ld_t;
  const bool vec_ok = AL;
  const float cf = R.c;
  auto wf = [=](float x, float, int e) -> double {
    if (x < tau || e == exclude) x = NEG_INF;
    return (double)term(x, m, cf);
  };
  return draw_chunk<TT, TT, false>(rp, rp, vec_ok, vec_ok, 0.f, c0, n, tl, wf, sm, ds);
}

__device__ __forceinline__ void write_fault(const Params& P, int b, int cu0, int k, int code) {
  for (int j = threadIdx.x; j <= k; j += WG) P.out[cu0 + j] = -1;
  const int d0 = cu0 - b;
  for (int j = threadIdx.x; j < k; j += WG) {
    if (P.p_at) P.p_at[d0 + j] = __builtin_nanf("");
    if (P.q_at) P.q_at[d0 + j] = __builtin_nanf("");
  }
  if (threadIdx.x == 0) {
    P.accepted[b] = -1;
    P.status[b] = code;
  }
}

// Helpers of a request wait for decision words exactly when this holds.
__device__ __forceinline__ bool has_helpers(const Params& P, const Req& R) {
  return P.H > 0 && !R.greedy && !R.bad_param &&
         (R.kind == SV_DRAFT_LOGITS || R.kind == SV_DRAFT_PROBS);
}

__device__ __forceinline__ void helpers_none(const Params& P, int b) {
  for (int e = threadIdx.x; e < P.nc * DEC_W; e += WG)
    put_w(P.dec + (int64_t)b * P.nc * DEC_W + e, F_NONE, 0u);
}

// ---------------------------------------------------------------------------
// finalizer: merge a request's statistics, scan, outputs, draws
// ---------------------------------------------------------------------------
struct FinShared {
  float M[64], Mq[64];
  double S[64], Sq[64];
  int g[64];
  float lx[64], sx[64], dlx[64];
  int x[64];
  float u[64];   // the request's uniforms, read with the draft ids
  float px[64], qx[64];   // p(x_j), q(x_j) handed to the last helper (mode 2)
  int a, code, mode, timeout;
};

template <typename TT, typename TD, bool AL>
__device__ __forceinline__ void finalize(const Params& P, int b, int cu0, int k, const Req& R, Smem& sm,
                         FinShared& fs, DrawShared& ds, uint32_t* stage) {
  const int nc = P.nc;
  const int d0 = cu0 - b;
  const int tid = threadIdx.x;
  const bool logits = R.kind == SV_DRAFT_LOGITS;
  const bool sampled = !R.greedy;
  // staged statistics: m and s (or argmax) of target rows 0..k (slots 0..k) and
  // draft rows 0..k-1 (slots k+1..2k), chunk-major within a row
  float* st_m = reinterpret_cast<float*>(stage);
  uint32_t* st_s = stage + (size_t)(2 * P.max_k + 1) * nc;

  // a poisoned workspace may hold stale hand-off words: take none of them
  const bool poisoned = ldu(P.ctl) != 0ull;
  if (tid == 0) fs.timeout = poisoned ? 1 : 0;
  if (tid < 64) {
    fs.x[tid] = (tid < k) ? P.drafts[d0 + tid] : -1;
    // uniforms exist for sampled requests only (the greedy entry passes none)
    fs.u[tid] = (!R.greedy && tid <= k) ? P.u[cu0 + tid] : 0.f;
  }
  __syncthreads();
  bool badtok_any = false;
  for (int i = 0; i < k; ++i) badtok_any |= (fs.x[i] < 0 || fs.x[i] >= P.vocab);

  if (!R.bad_param && !poisoned) {
    // wait for, stage and consume every word the request's producers published
    // (also when a draft id is out of range: the statistics were still written)
    const int nA = (k + 1) * nc;
    const int nB = logits ? k * nc : 0;
    const int rxw = sampled ? ((R.kind == SV_DRAFT_LOGITS || R.kind == SV_DRAFT_PROBS) ? 3 : 2) : 0;
    const int nC = k * rxw;
    int to = 0;
    for (int w = tid; w < nA + nB + nC; w += WG) {
      u64* src;
      int slot = -1, c = 0, f = 0, jr = 0;
      if (w < nA) {
        jr = w / nc;
        c = w - jr * nc;
        slot = jr;
        src = P.cst + ((int64_t)(cu0 + jr) * nc + c);
      } else if (w < nA + nB) {
        const int w2 = w - nA;
        jr = w2 / nc;
        c = w2 - jr * nc;
        slot = k + 1 + jr;
        src = P.dst + ((int64_t)(d0 + jr) * nc + c);
      } else {
        const int w3 = w - nA - nB;
        jr = w3 / rxw;
        f = w3 % rxw;
        if (fs.x[jr] < 0 || fs.x[jr] >= P.vocab) continue;   // never written
        src = P.rx + (int64_t)(cu0 + jr) * 3 + f;
      }
      const u64 v = take_w(src);
      if (!(hi32(v) & TAG)) to = 1;
      const uint32_t pay = lo32(v);
      if (slot >= 0) {
        st_m[slot * nc + c] = __uint_as_float(pay);
        st_s[slot * nc + c] = hi32(v) & ~TAG;
      } else if (f == 0) {
        fs.lx[jr] = __uint_as_float(pay);
      } else if (f == 1) {
        fs.sx[jr] = __uint_as_float(pay);
      } else {
        fs.dlx[jr] = __uint_as_float(pay);
      }
    }
    if (to) {
      atomicOr(&fs.timeout, 1);
      poison(P.ctl);
    }
  }
  __syncthreads();

  // staged rows (target rows 0..k, then draft rows 0..k-1), 16 lanes per row
  // (one DPP row): the row max; for sampled rows each chunk sum scaled to the
  // row max, in place, and the fp64 total of the scaled sums (lane-strided
  // partial sums, then a fixed butterfly over the 16 lanes); for greedy rows
  // the lowest chunk that holds the max
  const bool staged = !R.bad_param && !badtok_any && !fs.timeout;
  const int nrows = (k + 1) + (logits ? k : 0);
  if (staged) {
    const int sub = tid & 15;
    for (int r = tid >> 4; r < nrows; r += WG / 16) {   // the same r in all 16 lanes of a row
      const float* mrow = st_m + r * nc;
      uint32_t* srow = st_s + r * nc;
      float Ml = NEG_INF;
      for (int c = sub; c < nc; c += 16) Ml = fmax3nan(Ml, mrow[c]);
      Ml = fmax3nan(Ml, dpp_f<DPP_XOR1>(Ml));
      Ml = fmax3nan(Ml, dpp_f<DPP_XOR2>(Ml));
      Ml = fmax3nan(Ml, dpp_f<DPP_HMIRROR>(Ml));
      const float Mr = fmax3nan(Ml, dpp_f<DPP_MIRROR>(Ml));
      if (sampled) {
        const bool fin = Mr > NEG_INF && Mr < POS_INF;
        double Sl = 0.0;
        for (int c = sub; c < nc; c += 16) {
          const float m = mrow[c];
          float v = 0.f;
          if (fin && m > NEG_INF) v = __uint_as_float(srow[c]) * term(m, Mr, R.c);
          srow[c] = __float_as_uint(v);
          Sl += (double)v;
        }
        Sl += dpp_d<DPP_XOR1>(Sl);
        Sl += dpp_d<DPP_XOR2>(Sl);
        Sl += dpp_d<DPP_HMIRROR>(Sl);
        Sl += dpp_d<DPP_MIRROR>(Sl);
        if (sub == 0) {
          if (r <= k) {
            fs.M[r] = Mr;
            fs.S[r] = Sl;
          } else {
            fs.Mq[r - k - 1] = Mr;
            fs.Sq[r - k - 1] = Sl;
          }
        }
      } else {
        int cl = INT32_MAX;
        for (int c = sub; c < nc; c += 16)
          if (cl == INT32_MAX && mrow[c] == Mr) cl = c;
        cl = min(cl, dpp_i<DPP_XOR1>(cl));
        cl = min(cl, dpp_i<DPP_XOR2>(cl));
        cl = min(cl, dpp_i<DPP_HMIRROR>(cl));
        cl = min(cl, dpp_i<DPP_MIRROR>(cl));
        if (sub == 0) {
          fs.M[r] = Mr;
          fs.g[r] = cl < nc ? cl * CHUNK + (int)srow[cl] : -1;
        }
      }
    }
  }
  __syncthreads();

  if (tid < 64) {
    const int j = tid;
    bool nonfin = false, empty = false, acc = false;
    float M = NEG_INF, Mq = NEG_INF;
    double S = 0.0, Sq = 0.0;
    int g = -1;
    if (j <= k && staged) {
      M = fs.M[j];
      if (R.greedy) g = fs.g[j];
      else S = fs.S[j];
      nonfin = (M != M) || M == POS_INF;
      empty = M == NEG_INF;
      if (logits && j < k) {
        Mq = fs.Mq[j];
        Sq = fs.Sq[j];
        nonfin = nonfin || (Mq != Mq) || Mq == POS_INF;
        empty = empty || Mq == NEG_INF;
      }
    }
    const int x = fs.x[j];
    double px = 0.0, qx = 0.0;
    const uint64_t m_pre = __ballot(nonfin || empty);
    if (j < k && m_pre == 0 && staged) {
      if (R.greedy) {
        acc = (x == g);
        px = acc ? 1.0 : 0.0;
        qx = 1.0;
      } else {
        const double ex = exp2(((double)fs.lx[j] - (double)M) * R.ce);   // e_x in row-max units
        px = ex / S;
        if (logits) {
          float dl = fs.dlx[j];
          if (R.filt && P.thr_d && dl < thr_of(P.thr_d, d0 + j)) dl = NEG_INF;
          qx = exp2(((double)dl - (double)Mq) * R.ce) / Sq;
        } else if (R.kind == SV_DRAFT_PROBS) {
          qx = (double)fs.dlx[j];
          if (!(qx >= 0.0 && qx < (double)POS_INF)) nonfin = true;
        } else {
          qx = 1.0;
        }
        if (R.kind == SV_DRAFT_MATCH) {
          // the row's own sample is x iff u*S falls in x's interval of the
          // running sum in token order: [mass before x, mass before x + e_x)
          const int cx = x / CHUNK;
          const float* mrow = st_m + j * nc;
          const uint32_t* srow = st_s + j * nc;
          double before = 0.0;
          for (int c = 0; c < cx; ++c) before += (double)__uint_as_float(srow[c]);
          if (mrow[cx] > NEG_INF)
            before += (double)(fs.sx[j] * term(mrow[cx], M, R.c));
          const double us = (double)fs.u[j] * S;
          acc = ex > 0.0 && before <= us && us < before + ex;
        } else {
          acc = (double)fs.u[j] * qx < px;
        }
      }
    }
    const uint64_t m_nf = __ballot(nonfin);
    const uint64_t m_em = __ballot(empty);
    const uint64_t m_acc = __ballot(acc && j < k);
    int code = SV_ROW_OK;
    if (R.bad_param) code = SV_ROW_BAD_PARAM;
    else if (badtok_any) code = SV_ROW_BAD_TOKEN;
    else if (fs.timeout) code = SV_ROW_INTERNAL;
    else if (m_nf) code = SV_ROW_NONFINITE;
    else if (m_em) code = SV_ROW_EMPTY;
    int a = (int)__builtin_ctzll(~m_acc);
    if (a > k) a = k;
    fs.M[j] = M; fs.Mq[j] = Mq; fs.S[j] = S; fs.Sq[j] = Sq;
    // mode 2 (a rejection under a logit or probability draft): the helpers
    // finish the request, and its last helper is the only writer of its outputs
    const bool resid = code == SV_ROW_OK && sampled && a < k &&
                       (R.kind == SV_DRAFT_LOGITS || R.kind == SV_DRAFT_PROBS);
    if (resid && j < k) {
      fs.px[j] = (float)px;
      fs.qx[j] = (float)qx;
    }
    if (code == SV_ROW_OK && !resid) {
      if (j < k) {
        if (P.p_at) P.p_at[d0 + j] = (float)px;
        if (P.q_at) P.q_at[d0 + j] = (float)qx;
      }
      if (j <= k) {
        int tok = -1;
        if (j < a) tok = x;
        else if (j == a && R.greedy) tok = g;
        if (j != a || R.greedy) P.out[cu0 + j] = tok;
      }
    }
    if (j == 0) {
      fs.code = code;
      fs.a = a;
      int mode = 0;   // 0 done, 1 draw from the target row here, 2 residual by the helpers
      if (code == SV_ROW_OK && sampled)
        mode = (a == k || R.kind == SV_DRAFT_ONEHOT || R.kind == SV_DRAFT_MATCH) ? 1 : 2;
      fs.mode = mode;
    }
  }
  __syncthreads();
  const int code = fs.code;
  const int a = fs.a;
  const int mode = fs.mode;
  if (code != SV_ROW_OK) {
    write_fault(P, b, cu0, k, code);
    // the helpers take a record even on a poisoned workspace, so they never wait long
    if (has_helpers(P, R)) helpers_none(P, b);
    return;
  }
  if (mode == 1) {
    const int row = cu0 + a;
    const float tau = (P.thr_t && R.filt) ? thr_of(P.thr_t, row) : NEG_INF;
    // one-hot rejection: the residual is p without the draft; a prefix-match
    // request commits row a's own sample, drawn with row a's uniform
    const bool match = R.kind == SV_DRAFT_MATCH;
    const int exclude = (a < k && !match) ? fs.x[a] : -1;
    // st_s holds the chunk sums already scaled to the row max
    const float* mrow = st_m + a * nc;
    const uint32_t* srow = st_s + a * nc;
    const float Ma = fs.M[a];
    const float sxa = exclude >= 0 ? fs.sx[a] : 0.f;
    const float cf = R.c;
    auto rc = [=](int c) { return (double)term(mrow[c], Ma, cf); };
    auto mass = [=](int c, bool ex) {
      if (!(mrow[c] > NEG_INF)) return 0.0;
      return ex ? (double)(sxa * term(mrow[c], Ma, cf)) : (double)__uint_as_float(srow[c]);
    };
    const int t = draw_target_row<TT, AL>(P, R, row, exclude, tau, (double)fs.u[match ? a : k],
                                          [=](int c) { return mrow[c]; }, mass, rc, sm, ds);
    if (tid == 0) P.out[row] = t;
    if (has_helpers(P, R)) helpers_none(P, b);
  } else if (mode == 2) {
    // "pending" until the last helper writes the request's outputs: if no helper
    // completes them (a wait ran out) the caller still sees INTERNAL.  Both
    // stores write through to memory, and the wave waits for them before the
    // records are posted, so the helper's stores, made after it takes a record,
    // land later.
    if (tid == 0) {
      st_agent(P.status + b, (int32_t)SV_ROW_INTERNAL);
      st_agent(P.accepted + b, (int32_t)-1);
      // both stores completed (the compiler's own wait insertion drops an
      // explicit wait that no later instruction of this wave depends on)
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
    __syncthreads();
    // every word of every record carries its own tag: no ordering among them
    if (tid < 2 * k) {
      const float v = tid < k ? fs.px[tid] : fs.qx[tid - k];
      put_w(P.pq + (int64_t)b * 2 * P.max_k + tid, 0u, __float_as_uint(v));
    }
    const u64 sp = (u64)__double_as_longlong(fs.S[a]);
    const u64 sq = (u64)__double_as_longlong(fs.Sq[a]);
    for (int e = tid; e < nc * DEC_W; e += WG) {
      const int c = e / DEC_W;
      const int f = e - c * DEC_W;
      uint32_t pay;
      switch (f) {
        case 0: pay = __float_as_uint(st_m[a * nc + c]); break;
        case 1: pay = logits ? __float_as_uint(st_m[(k + 1 + a) * nc + c]) : 0u; break;
        case 2: pay = (uint32_t)sp; break;
        case 3: pay = (uint32_t)(sp >> 32); break;
        case 4: pay = (uint32_t)sq; break;
        case 5: pay = (uint32_t)(sq >> 32); break;
        case 6: pay = __float_as_uint(fs.M[a]); break;
        default: pay = __float_as_uint(fs.Mq[a]); break;
      }
      put_w(P.dec + (int64_t)b * nc * DEC_W + e, f == 0 ? (uint32_t)a : 0u, pay);
    }
  }
  if (tid == 0 && mode != 2) {
    P.accepted[b] = a;
    P.status[b] = SV_ROW_OK;
  }
}

// ---------------------------------------------------------------------------
// helpers: residual max(0, p - q) at the first rejection
// ---------------------------------------------------------------------------
struct ResCtx {
  float c;         // log2(e) / T of the request
  float mp, mq;    // chunk maxima of target and draft
  double sp, sq;   // per-chunk scale R_c / S of target and draft
  float taup, tauq;
};

// Residual weight of one token from its target value lp and draft value lq
// (logit, or probability for a probability draft).
template <bool LOGITS>
__device__ __forceinline__ double resid_elem(float lp, float lq, const ResCtx& X) {
  if (lp < X.taup) lp = NEG_INF;
  const double p = (double)term(lp, X.mp, X.c) * X.sp;
  double q;
  if (LOGITS) {
    if (lq < X.tauq) lq = NEG_INF;
    q = (double)term(lq, X.mq, X.c) * X.sq;
  } else {
    q = (double)lq;
  }
  const double w = p - q;
  return w > 0.0 ? w : 0.0;
}

__device__ __forceinline__ void res_ctx(const Params& P, const Req& R, const Setup& su, float mp,
                                        float mq, int trow, int drow, ResCtx& X) {
  X.c = R.c;
  X.mp = (mp > NEG_INF) ? mp : 0.f;
  X.sp = (mp > NEG_INF) ? scale_d(mp, su.Mp, R.ce) / su.Sp : 0.0;
  X.taup = (P.thr_t && R.filt) ? thr_of(P.thr_t, trow) : NEG_INF;
  X.mq = 0.f;
  X.sq = 0.0;
  X.tauq = NEG_INF;
  if (R.kind == SV_DRAFT_LOGITS) {
    X.mq = (mq > NEG_INF) ? mq : 0.f;
    X.sq = (mq > NEG_INF) ? scale_d(mq, su.Mq, R.ce) / su.Sq : 0.0;
    X.tauq = (P.thr_d && R.filt) ? thr_of(P.thr_d, drow) : NEG_INF;
  }
}

struct HelpShared {
  u64 rec[DEC_W];
  float pq[2 * 64];   // the last helper's copy of p(x_j), q(x_j)
  int timeout, bad;
};

// The outputs of a request that rejected under a logit or probability draft,
// written by its last helper alone (the drawing helper writes the token at the
// stop position): accepted drafts, -1 past the stop position, p and q at the
// drafts, the accepted count and the status.
__device__ __forceinline__ void finish_outputs(const Params& P, int b, int cu0, int k, int a,
                                               const HelpShared& hs) {
  const int d0 = cu0 - b;
  for (int j = threadIdx.x; j <= k; j += WG) {
    if (j < a) P.out[cu0 + j] = P.drafts[d0 + j];
    else if (j > a) P.out[cu0 + j] = -1;
  }
  for (int j = threadIdx.x; j < k; j += WG) {
    if (P.p_at) P.p_at[d0 + j] = hs.pq[j];
    if (P.q_at) P.q_at[d0 + j] = hs.pq[k + j];
  }
  if (threadIdx.x == 0) {
    st_agent(P.accepted + b, (int32_t)a);
    st_agent(P.status + b, (int32_t)SV_ROW_OK);
  }
}

template <typename TT, typename TD, bool AL>
__device__ __forceinline__ void helper(const Params& P, int b, int cu0, int k, int c, Smem& sm,
                                       DrawShared& ds, HelpShared& hs) {
  const int nc = P.nc;
  const Req R = load_req(P, b);
  if (!has_helpers(P, R)) return;
  const bool logits = R.kind == SV_DRAFT_LOGITS;
  // the decision record: one word per thread, all taken at once
  if (threadIdx.x < DEC_W) hs.rec[threadIdx.x] = take_w(P.dec + ((int64_t)b * nc + c) * DEC_W + threadIdx.x);
  __syncthreads();
  const bool last = c == nc - 1;
  {
    bool to = false;
#pragma unroll
    for (int f = 0; f < DEC_W; ++f) to = to || !(hi32(hs.rec[f]) & TAG);
    if (to) {
      // the finalizer's outputs (or its pending INTERNAL) stand: nothing is written here
      if (threadIdx.x == 0) poison(P.ctl);
      return;
    }
  }
  if (hi32(hs.rec[0]) & F_NONE) return;
  if (last) {
    // p(x_j) and q(x_j) of the request, for the outputs this helper writes
    if (threadIdx.x == 0) hs.timeout = 0;
    __syncthreads();
    if (threadIdx.x < 2 * k) {
      const u64 v = take_w(P.pq + (int64_t)b * 2 * P.max_k + threadIdx.x);
      if (!(hi32(v) & TAG)) atomicOr(&hs.timeout, 1);
      hs.pq[threadIdx.x] = __uint_as_float(lo32(v));
    }
    __syncthreads();
    if (hs.timeout) {
      if (threadIdx.x == 0) poison(P.ctl);
      write_fault(P, b, cu0, k, SV_ROW_INTERNAL);
      return;
    }
  }
  Setup su;
  su.Sp = __longlong_as_double((long long)((u64)lo32(hs.rec[2]) | ((u64)lo32(hs.rec[3]) << 32)));
  su.Sq = __longlong_as_double((long long)((u64)lo32(hs.rec[4]) | ((u64)lo32(hs.rec[5]) << 32)));
  su.Mp = __uint_as_float(lo32(hs.rec[6]));
  su.Mq = __uint_as_float(lo32(hs.rec[7]));
  su.a = (int)(hi32(hs.rec[0]) & 63u);
  const float cmp = __uint_as_float(lo32(hs.rec[0]));   // this chunk's maxima
  const float cmq = logits ? __uint_as_float(lo32(hs.rec[1])) : 0.f;
  const int a = su.a;
  if (a < 0 || a >= k) {   // cannot happen after a fresh decision; never index with it
    if (threadIdx.x == 0) poison(P.ctl);
    if (last) write_fault(P, b, cu0, k, SV_ROW_INTERNAL);
    return;
  }
  const int trow = cu0 + a;
  const int drow = cu0 - b + a;
  const TT* tp = target_rows<TT>(P, R.pen) + (int64_t)trow * P.ld_t;
  const TD* dp = (const TD*)P.draft + (int64_t)drow * P.ld_d;
  const bool tvec = AL;
  const bool dvec = AL;
  const bool probs = R.kind == SV_DRAFT_PROBS;
  const float qfill = probs ? 0.f : NEG_INF;
  double W;
  int anybad;
  ResCtx X;
  // the chunk is requested first; the weights' context is computed while it loads
  const int c0 = c * CHUNK;
  const int n = min(CHUNK, P.vocab - c0);
  Seg<TT> sp;
  Seg<TD> sq;
  load_contig<TT>(tp + c0, n, tvec, NEG_INF, sp);
  load_contig<TD>(dp + c0, n, dvec, qfill, sq);
  const double u = (double)P.u[cu0 + k];   // arrives with the chunk
  res_ctx(P, R, su, cmp, cmq, trow, drow, X);
  // the chunk's residual mass as the total of a block scan of the segment
  // sums: the scan, the segment sums and the last positive elements are kept
  // for the draw, which then evaluates only the winning segment again
  auto wl = [=](float lp, float lq, int) -> double { return resid_elem<true>(lp, lq, X); };
  auto wpr = [=](float lp, float lq, int) -> double { return resid_elem<false>(lp, lq, X); };
  double own, excl, incl;
  {
    bool bad = false;
    if (logits) {
      own = seg_weights<TT, TD, true>(sp, sq, c0, wl);
    } else {
      own = seg_weights<TT, TD, true>(sp, sq, c0, wpr);
#pragma unroll
      for (int i = 0; i < EPT; ++i) {
        const float lq = sq.at(i);
        bad = bad || !(lq >= 0.f && lq < POS_INF);
      }
    }
    block_scan_total_d(own, excl, incl, W, sm);
    anybad = logits ? 0 : block_max_i(bad ? 1 : 0, sm);   // logits are checked by the producers
  }
  if (nc <= PEER_MAX) {
    // every helper sends its chunk's mass to every other helper of the request
    // and takes theirs, so each picks the chunk itself; the one holding the
    // chosen chunk draws from the registers it already has.  A helper waits here
    // for helpers launched after it: a request's helpers are launched together,
    // at most one request's set is partly resident at a time, and everything
    // else finishes without waiting for helpers, so that set is completed.
    u64* row = P.res + (int64_t)b * nc * nc;
    const uint32_t fl = anybad ? F_BAD : 0u;
    const uint32_t wv = __float_as_uint((float)W);
    for (int t = threadIdx.x; t < nc; t += WG)
      if (t != c) put_w(row + (int64_t)t * nc + c, fl, wv);
    if (threadIdx.x == 0) {
      hs.bad = anybad;
      hs.timeout = 0;
    }
    __syncthreads();
    int to = 0, bd = 0;
    for (int t = threadIdx.x; t < nc; t += WG) {
      if (t == c) {
        ds.E[t] = (double)(float)W;
        continue;
      }
      const u64 v = take_w(row + (int64_t)c * nc + t);
      if (!(hi32(v) & TAG)) to = 1;
      if (hi32(v) & F_BAD) bd = 1;
      ds.E[t] = (double)__uint_as_float(lo32(v));
    }
    if (to) {
      atomicOr(&hs.timeout, 1);
      poison(P.ctl);
    }
    if (bd) atomicOr(&hs.bad, 1);
    __syncthreads();
    if (hs.timeout || hs.bad) {
      if (last) write_fault(P, b, cu0, k, hs.timeout ? SV_ROW_INTERNAL : SV_ROW_NONFINITE);
      return;
    }
    if (last) finish_outputs(P, b, cu0, k, a, hs);
    if (!pick_chunk(nc, u, ds)) {
      if (last) {
        const float tau = (P.thr_t && R.filt) ? thr_of(P.thr_t, trow) : NEG_INF;
        const u64* cw = P.cst + (int64_t)trow * nc;
        const float Mp = su.Mp;
        const double ce = R.ce;
        auto cm = [=](int cc) { return __uint_as_float(lo32(ld_agent(cw + cc))); };
        auto rc = [=](int cc) { return scale_d(cm(cc), Mp, ce); };
        auto mass = [=](int cc, bool) {
          const float m = cm(cc);
          if (!(m > NEG_INF)) return 0.0;
          return (double)__uint_as_float(hi32(ld_agent(cw + cc)) & ~TAG) * scale_d(m, Mp, ce);
        };
        const int t = draw_target_row<TT, AL>(P, R, trow, -1, tau, u, cm, mass, rc, sm, ds);
        if (threadIdx.x == 0) P.out[trow] = t;
      }
      return;
    }
    if (ds.chunk != c) return;
    const double tl = ds.tl;
    int t;
    if (logits)
      t = draw_scanned<TT, TD, true>(sp, sq, qfill, c0, n, tl, wl, own, excl, incl, sm, ds);
    else
      t = draw_scanned<TT, TD, true>(sp, sq, qfill, c0, n, tl, wpr, own, excl, incl, sm, ds);
    if (threadIdx.x == 0) P.out[trow] = t;
    return;
  }
  if (!last) {
    if (threadIdx.x == 0)
      put_w(P.res + (int64_t)b * nc + c, anybad ? F_BAD : 0u, __float_as_uint((float)W));
    return;
  }
  // last helper: collect the other chunks' residual masses, pick, draw
  if (threadIdx.x == 0) {
    hs.bad = anybad;
    hs.timeout = 0;
  }
  __syncthreads();
  int to = 0, bd = 0;
  for (int cc = threadIdx.x; cc < nc - 1; cc += WG) {
    const u64 v = take_w(P.res + (int64_t)b * nc + cc);
    if (!(hi32(v) & TAG)) to = 1;
    if (hi32(v) & F_BAD) bd = 1;
    ds.E[cc] = (double)__uint_as_float(lo32(v));
  }
  if (threadIdx.x == 0) ds.E[nc - 1] = (double)(float)W;
  if (to) {
    atomicOr(&hs.timeout, 1);
    poison(P.ctl);
  }
  if (bd) atomicOr(&hs.bad, 1);
  __syncthreads();
  if (hs.timeout) {
    write_fault(P, b, cu0, k, SV_ROW_INTERNAL);
    return;
  } else if (hs.bad) {
    write_fault(P, b, cu0, k, SV_ROW_NONFINITE);
    return;
  }
  finish_outputs(P, b, cu0, k, a, hs);
  if (!pick_chunk(nc, u, ds)) {
    // residual mass is exactly zero: draw from p of the rejected row, using the
    // row's chunk statistics (their payloads stay in the words after consumption)
    const float tau = (P.thr_t && R.filt) ? thr_of(P.thr_t, trow) : NEG_INF;
    const u64* cw = P.cst + (int64_t)trow * nc;
    const float Mp = su.Mp;
    const double ce = R.ce;
    auto cm = [=](int cc) { return __uint_as_float(lo32(ld_agent(cw + cc))); };
    auto rc = [=](int cc) { return scale_d(cm(cc), Mp, ce); };
    auto mass = [=](int cc, bool) {
      const float m = cm(cc);
      if (!(m > NEG_INF)) return 0.0;
      return (double)__uint_as_float(hi32(ld_agent(cw + cc)) & ~TAG) * scale_d(m, Mp, ce);
    };
    const int t = draw_target_row<TT, AL>(P, R, trow, -1, tau, u, cm, mass, rc, sm, ds);
    if (threadIdx.x == 0) P.out[trow] = t;
  } else {
    const int ch = ds.chunk;
    const double tl = ds.tl;
    // the chosen chunk's maxima: from the decision payloads left in the words
    const u64* dw = P.dec + ((int64_t)b * nc + ch) * DEC_W;
    const float mp = __uint_as_float(lo32(ld_agent(dw)));
    const float mq = logits ? __uint_as_float(lo32(ld_agent(dw + 1))) : 0.f;
    ResCtx Xc;
    res_ctx(P, R, su, mp, mq, trow, drow, Xc);
    const int cc0 = ch * CHUNK;
    const int cn = min(CHUNK, P.vocab - cc0);
    int t;
    if (logits) {
      auto wf = [=](float lp, float lq, int) -> double { return resid_elem<true>(lp, lq, Xc); };
      t = draw_chunk<TT, TD, true>(tp, dp, tvec, dvec, qfill, cc0, cn, tl, wf, sm, ds);
    } else {
      auto wf = [=](float lp, float lq, int) -> double { return resid_elem<false>(lp, lq, Xc); };
      t = draw_chunk<TT, TD, true>(tp, dp, tvec, dvec, qfill, cc0, cn, tl, wf, sm, ds);
    }
    if (threadIdx.x == 0) P.out[trow] = t;
  }
}

// ---------------------------------------------------------------------------
// k_verify: block index -> role
//   The producers of every request come first, request by request in launch
//   order ((max_k+1) * ns workgroups per request: row j, strip s), then the
//   helpers, H workgroups per request in the same order.  The sampled requests
//   with draft rows -- the only ones whose helpers have work -- are launched
//   first, so their finalizers decide while later requests still stream, and
//   their helpers, dispatched as the last producers start, find the decision
//   posted or close to it instead of holding a slot through the streaming.
// ---------------------------------------------------------------------------
// ---------------------------------------------------------------------------
// launch order of the requests
// ---------------------------------------------------------------------------
// Requests are laid out in the grid by class: sampled requests with draft rows
// (their rejection needs the helpers) first, other sampled requests next,
// greedy ones last, each class in request order.  The work after a request's
// last producer (merge, draws) then overlaps later requests' producers, and
// the call ends on the cheapest chains.
//
// In a batch of up to 64 requests every wave finds the request at its launch
// position on its own: one request per lane, its offsets, temperature and
// draft kind loaded together (one round trip), classes counted by ballots and
// DPP scans.  A larger batch (kernels instantiated with E = 16) has k_order
// write the table once per call: sixteen requests per lane looked up in every
// workgroup cost more than the table's launch as soon as the grid holds
// thousands of workgroups.
// A request is valid when its offsets pass req_valid and its first draft row
// cu[b] - b is not below any earlier request's cu[e] - e.  That also puts cu[b]
// above every earlier offset, so neither the target rows nor the draft rows of
// valid requests overlap (an earlier request with no rows, or offsets that go
// back, would otherwise let the next draft rows reach into an earlier
// request's, and two requests would publish to the same hand-off words).
__device__ __forceinline__ int first_drow(int cu_i, int i) {   // cu[i] - i, clamped
  return (int)max((long long)cu_i - i, (long long)INT32_MIN);
}

struct ReqPos {
  int b, cu0, cu1;
  int cls;        // launch class: 0 sampled with draft rows, 1 other sampled, 2 greedy
  bool valid;
};

__device__ __forceinline__ int wave_scan_add(int x) {   // inclusive, over the wave
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false);   // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false);   // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false);   // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false);   // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);   // row_bcast:15
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);   // row_bcast:31
  return x;
}
__device__ __forceinline__ int wave_scan_max(int x) {   // inclusive, over the wave
  x = max(x, __builtin_amdgcn_update_dpp(INT32_MIN, x, 0x111, 0xf, 0xf, false));
  x = max(x, __builtin_amdgcn_update_dpp(INT32_MIN, x, 0x112, 0xf, 0xf, false));
  x = max(x, __builtin_amdgcn_update_dpp(INT32_MIN, x, 0x114, 0xf, 0xf, false));
  x = max(x, __builtin_amdgcn_update_dpp(INT32_MIN, x, 0x118, 0xf, 0xf, false));
  x = max(x, __builtin_amdgcn_update_dpp(INT32_MIN, x, 0x142, 0xa, 0xf, false));
  x = max(x, __builtin_amdgcn_update_dpp(INT32_MIN, x, 0x143, 0xc, 0xf, false));
  return x;
}

template <int E>
__device__ __forceinline__ ReqPos req_at(const Params& P, int pos) {
  if constexpr (E > 1) {   // batches of more than 64: the table k_order wrote
    const int32_t* r = P.order + 4 * pos;
    ReqPos R;
    R.b = ldu(r);
    R.cu0 = ldu(r + 1);
    R.cu1 = ldu(r + 2);
    const int w = ldu(r + 3);
    R.cls = w & 3;
    R.valid = (w & 4) != 0;
    return R;
  }
  const int lane = threadIdx.x & 63;
  const int B = P.batch;
  const int i0 = lane * E;
  int lo[E + 1], cl[E];
#pragma unroll
  for (int e = 0; e <= E; ++e) lo[e] = P.cu[min(i0 + e, B)];
  if (!P.greedy_entry) {
    float T[E];
    int kd[E];
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int i = min(i0 + e, B - 1);
      T[e] = P.temp[i];
      kd[e] = P.kind[i];
    }
#pragma unroll
    for (int e = 0; e < E; ++e)
      cl[e] = (i0 + e >= B) ? 3 : !(T[e] >= FLT_MIN) ? 2
              : (kd[e] == SV_DRAFT_LOGITS || kd[e] == SV_DRAFT_PROBS) ? 0 : 1;
  } else {
#pragma unroll
    for (int e = 0; e < E; ++e) cl[e] = (i0 + e >= B) ? 3 : 2;
  }
  // class counts: totals and this lane's exclusive prefix
  int c0 = 0, c1 = 0, c2 = 0;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    c0 += cl[e] == 0;
    c1 += cl[e] == 1;
    c2 += cl[e] == 2;
  }
  const int s0 = wave_scan_add(c0), s1 = wave_scan_add(c1), s2 = wave_scan_add(c2);
  const int n0 = __builtin_amdgcn_readlane(s0, 63), n1 = __builtin_amdgcn_readlane(s1, 63);
  const int tc = pos < n0 ? 0 : (pos < n0 + n1 ? 1 : 2);
  const int r = pos - (tc >= 1 ? n0 : 0) - (tc == 2 ? n1 : 0);
  const int cnt = tc == 0 ? c0 : (tc == 1 ? c1 : c2);
  const int excl = (tc == 0 ? s0 : (tc == 1 ? s1 : s2)) - cnt;
  const bool mine = r >= excl && r < excl + cnt;
  // the lane's entry of rank r within class tc
  int ei = 0, seen = excl;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    if (cl[e] == tc) {
      if (seen == r) ei = e;
      ++seen;
    }
  }
  // offsets must not go back: the running max of cu[i] - i over the requests
  // before that entry
  int mloc = INT32_MIN, run_at = INT32_MIN;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    if (e == ei) run_at = mloc;
    mloc = (i0 + e < B) ? max(mloc, first_drow(lo[e], i0 + e)) : mloc;
  }
  const int minc = wave_scan_max(mloc);
  const int before = __builtin_amdgcn_update_dpp(INT32_MIN, minc, 0x138, 0xf, 0xf, false);  // wave_shr:1
  run_at = max(run_at, before);
  int c_lo = 0, c_hi = 0;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    if (e == ei) {
      c_lo = lo[e];
      c_hi = lo[e + 1];
    }
  }
  const uint64_t m = __ballot(mine);
  const int src = m ? (int)__builtin_ctzll(m) : 0;   // classes partition the batch: m != 0
  ReqPos R;
  R.b = __builtin_amdgcn_readlane(i0 + ei, src);
  R.cu0 = __builtin_amdgcn_readlane(c_lo, src);
  R.cu1 = __builtin_amdgcn_readlane(c_hi, src);
  const int ra = __builtin_amdgcn_readlane(run_at, src);
  R.cls = tc;
  R.valid = R.cu0 >= 0 && R.cu0 - R.b >= ra && req_valid(P, R.b, R.cu0, R.cu1, R.cu1 - R.cu0 - 1);
  return R;
}

// Whether request b's offsets are valid, the verdict req_at gives for it: one
// wave-level load of the offsets for the largest cu[i] - i before b.
template <int E>
__device__ __forceinline__ bool offsets_ok(const Params& P, int b, int cu0, int cu1) {
  if constexpr (E > 1) return ldu(P.okb + b) != 0;   // k_order's verdict
  const int i0 = (threadIdx.x & 63) * E;
  int m = INT32_MIN;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int v = P.cu[min(i0 + e, P.batch)];
    if (i0 + e < b) m = max(m, first_drow(v, i0 + e));
  }
  const int ra = __builtin_amdgcn_readlane(wave_scan_max(m), 63);
  return cu0 >= 0 && cu0 - b >= ra && req_valid(P, b, cu0, cu1, cu1 - cu0 - 1);
}

// The requests in launch order, once per call, for batches of more than 64
// requests (one workgroup of 1,024 threads, thread t for request t): the
// classes req_at sorts by (0 sampled with draft rows, 1 other sampled, 2
// greedy; request order within a class), each request's place in that order,
// and its offsets verdict (cu[t] - t at or above every earlier one, and the
// checks of req_valid) -- what req_at and offsets_ok find in place for small
// batches.  The workgroups of the later kernels then find their request with
// one scalar load.
__global__ __launch_bounds__(1024) void k_order(const Params P) {
  __shared__ int wsum[3][16];
  __shared__ int wmax[16];
  const int t = threadIdx.x;
  const int lane = t & 63, wv = t >> 6;
  const int B = P.batch;
  int cl = 3, cu0 = 0, cu1 = 0, fd = INT32_MIN;
  if (t < B) {
    cu0 = P.cu[t];
    cu1 = P.cu[t + 1];
    if (P.greedy_entry) {
      cl = 2;
    } else {
      const float T = P.temp[t];
      const int kd = P.kind[t];
      cl = !(T >= FLT_MIN) ? 2 : (kd == SV_DRAFT_LOGITS || kd == SV_DRAFT_PROBS) ? 0 : 1;
    }
    fd = first_drow(cu0, t);
  }
  const int s0 = wave_scan_add(cl == 0 ? 1 : 0);
  const int s1 = wave_scan_add(cl == 1 ? 1 : 0);
  const int s2 = wave_scan_add(cl == 2 ? 1 : 0);
  const int mx = wave_scan_max(fd);
  const int before = __builtin_amdgcn_update_dpp(INT32_MIN, mx, 0x138, 0xf, 0xf, false);  // wave_shr:1
  if (lane == 63) {
    wsum[0][wv] = s0;
    wsum[1][wv] = s1;
    wsum[2][wv] = s2;
    wmax[wv] = mx;
  }
  __syncthreads();
  int b0 = 0, b1 = 0, b2 = 0, n0 = 0, n1 = 0, ra = before;
  for (int q = 0; q < 16; ++q) {
    if (q < wv) {
      b0 += wsum[0][q];
      b1 += wsum[1][q];
      b2 += wsum[2][q];
      ra = max(ra, wmax[q]);
    }
    n0 += wsum[0][q];
    n1 += wsum[1][q];
  }
  if (t < B) {
    const int pos = cl == 0 ? b0 + s0 - 1 : cl == 1 ? n0 + b1 + s1 - 1 : n0 + n1 + b2 + s2 - 1;
    const bool valid = cu0 >= 0 && cu0 - t >= ra && req_valid(P, t, cu0, cu1, cu1 - cu0 - 1);
    *reinterpret_cast<int4*>(P.order + 4 * pos) = make_int4(t, cu0, cu1, cl | (valid ? 4 : 0));
    P.okb[t] = valid ? 1 : 0;
  }
}

template <typename TT, typename TD, bool AL, int E>
__global__ __launch_bounds__(WG, 4) void k_verify(const Params P) {
  __shared__ Smem sm;
  __shared__ FinShared fs;
  __shared__ DrawShared ds;
  __shared__ HelpShared hs;
  __shared__ ProdShared ps;
  extern __shared__ uint32_t stage[];
  const int Pw = (P.max_k + 1) * P.ns;
  long long id = blockIdx.x;
  if (P.dsplit) {   // draft strips first
    const long long nd = (long long)P.batch * P.max_k * P.ns;
    if (id < nd) {
      const int Pd = P.max_k * P.ns;
      const int b = (int)(id / Pd);
      const int loc = (int)(id - (long long)b * Pd);
      const int j = loc / P.ns;
      const int s = loc - j * P.ns;
      // scalar loads decide which requests have draft-logit rows; only those
      // pay the vector lookup that checks the offsets
      const Req R = load_req(P, b);
      const int cu0 = ldu(P.cu + b), cu1 = ldu(P.cu + b + 1);
      if (R.greedy || R.bad_param || R.kind != SV_DRAFT_LOGITS || j >= cu1 - cu0 - 1) return;
      if (!offsets_ok<E>(P, b, cu0, cu1)) return;
      // the threshold kernel wrote this row's word in this call (same
      // conditions), and published its statistics when it says so
      if (R.filt && P.thr_d && hi32(ldu(P.thr_d + (cu0 - b + j))) == THR_PUBLISHED) return;
      Buf<TT, TD> A;
      issue_task<TT, TD, AL>((const TT*)nullptr, (const TD*)P.draft + (int64_t)(cu0 - b + j) * P.ld_d,
                             true, s * P.S, P.vocab, A);
      produce_draft<TT, TD, AL>(P, R, b, cu0, j, s, ps, A);
      return;
    }
    id -= nd;
  }
  const long long np = (long long)P.batch * Pw;   // producer workgroups
  if (id >= np) {   // helper of the request at position hpos, chunk c
    const int hpos = (int)((id - np) / P.H);
    const int c = (int)(id - np - (long long)hpos * P.H);
    const ReqPos Q = req_at<E>(P, hpos);
    // only requests with draft rows (class 0) have helper work
    if (Q.valid && Q.cls == 0) helper<TT, TD, AL>(P, Q.b, Q.cu0, Q.cu1 - Q.cu0 - 1, c, sm, ds, hs);
    return;
  }
  const int per = (int)(id / Pw);
  const int loc = (int)(id - (long long)per * Pw);
  const int j = loc / P.ns;
  const int s = loc - j * P.ns;
  const ReqPos Q = req_at<E>(P, per);
  const int b = Q.b;
  const int cu0 = Q.cu0;
  const int k = Q.cu1 - cu0 - 1;
  if (!Q.valid) {
    if (j == 0 && s == 0 && threadIdx.x == 0) {
      P.accepted[b] = -1;
      P.status[b] = SV_ROW_BAD_K;
    }
    return;
  }
  if (j > k) return;
  // a filtered row whose statistics the threshold kernel published (it wrote
  // the row's word in this call under the same conditions) needs no strip;
  // the strip's first chunk is requested before the request's parameters
  const bool pub = P.thr_t && hi32(ldu(P.thr_t + cu0 + j)) == THR_PUBLISHED;
  Buf<TT, TD> A;
  if (!pub)
    issue_task<TT, TD, AL>(target_rows<TT>(P, pen_of(P, b)) + (int64_t)(cu0 + j) * P.ld_t,
                           (const TD*)nullptr, false, s * P.S, P.vocab, A);
  const Req R = load_req(P, b);
  if (!R.bad_param && !(pub && R.filt && !R.greedy)) {
    if (pub)   // a word left from an earlier call: the strip runs after all
      issue_task<TT, TD, AL>(target_rows<TT>(P, R.pen) + (int64_t)(cu0 + j) * P.ld_t,
                             (const TD*)nullptr, false, s * P.S, P.vocab, A);
    produce<TT, TD, AL>(P, R, b, cu0, k, j, s, ps, A);
  }
  if (j == k && s == P.ns - 1) finalize<TT, TD, AL>(P, b, cu0, k, R, sm, fs, ds, stage);
}

// ---------------------------------------------------------------------------
// k_thresh: top-k / top-p thresholds, one workgroup of 1,024 threads per
// filtered row
// ---------------------------------------------------------------------------
// A row's threshold is the value of a radix select over order-preserving
// 32-bit keys of its values (-0 folded into +0), 8 key bits per level: 2
// levels for bf16 rows, whose keys carry 16 bits, 4 for fp32.  Top-k counts
// values per digit; top-p sums their masses exp2((v - M) c) rounded to integer
// multiples of 2^-40, so that every order of summation gives the same totals.
//
// A row of up to 131,072 bf16 or 65,536 fp32 values, 16-byte aligned, is read
// from HBM once and kept in registers (16 128-bit words per thread); every
// later pass runs from there.  Longer or unaligned rows are read again for
// each pass.  The passes are VALU-bound (a wave64 vector instruction takes 4
// cycles), so the full-row work is kept to a few instructions per value:
//
// * top-k (K <= 1,024): each wave's r-th largest thread maximum, r =
//   ceil(K / 16), found by a ballot binary search over the key bits, and the
//   smallest of the 16 is a lower bound of the K-th largest value; one compare
//   pass appends every value at or above it to a list in LDS, and the select
//   runs on the list;
// * top-p without top-k: one pass sums the integer masses per thread in fp64
//   for the total Z (fp32 sums of the eight values of a 128-bit word, added
//   in fp64 in a fixed order: deterministic, within about 1e-7), and adds
//   every term into one of 64 bins by its binary exponent, as its top 13
//   significant bits (integer LDS atomics, so within 2^-12 of the sum);
//   the bins below the smallest exponent whose tail, taken 1% heavier,
//   weighs less than (1 - P) Z cannot hold the cut, so a compare pass against
//   a value safely below that exponent fills the list, and the select runs on
//   the list;
// * top-p after top-k: every value of the top-k set is on the list already.
//
// Both selects on a list give the threshold of the full row: every value down
// to the cut is on the list, so the digit where the sum from the top reaches
// the goal is the same.  Each wave appends to a segment of its own, its count
// kept in registers.  A row whose list would overflow a segment, or whose
// bound is -inf, takes full-row radix passes instead.  A level's histogram has
// HCOPY copies, one per lane of a half wave, so lanes of one LDS atomic share
// an address only when they are 32 apart and agree on the digit (a list of at
// most LIST_SMALL entries adds into one copy); one wave then picks the digit
// from suffix sums of the merged bins.
//
// A threshold found on a list also gives the row's chunk statistics: every
// kept value is on the list, so the workgroup publishes them in the words the
// verify kernel's producers would write (publish_stats) and marks the row's
// threshold word; that kernel then leaves the row alone, which is read once.
constexpr int TW = 1024;          // threads of a threshold workgroup
constexpr int TNW = TW / 64;
constexpr int THR_NL = 16;        // 128-bit words per thread of a row kept in registers
constexpr int HCOPY = 32;         // histogram copies
constexpr int LIST_BYTES = 90112; // LDS for the candidates of a row
// List entries: the value's bits (-0 folded into +0) and its place.  bf16: 32
// bits, the value's upper half over its place within its wave's share of the
// row (word i, lane, value h: 13 bits; the wave is the list segment's); fp32:
// 64 bits, the value's bits below the element index.
template <typename T> struct LE;
template <> struct LE<uint16_t> {
  using E = uint32_t;
  static constexpr unsigned CAP = LIST_BYTES / 4;
  // element e = (i * TW + wave * 64 + lane) * 8 + h lives at (i, lane, h);
  // bits: a bf16 value's fp32 bits (lower half zero)
  __device__ static E make(uint32_t bits, int e) {
    return bits | ((((uint32_t)e >> 4) & ~511u) | ((uint32_t)e & 511u));
  }
  __device__ static uint32_t bits(E en) { return en & 0xffff0000u; }
  __device__ static int index(E en, int wave) {
    const uint32_t l = en & 0xffffu;
    return (int)((l >> 9) * (TW * 8) + (uint32_t)wave * 512u + (l & 511u));
  }
};
template <> struct LE<float> {
  using E = unsigned long long;
  static constexpr unsigned CAP = LIST_BYTES / 8;
  __device__ static E make(uint32_t bits, int e) { return ((E)(uint32_t)e << 32) | bits; }
  __device__ static uint32_t bits(E en) { return (uint32_t)en; }
  __device__ static int index(E en, int) { return (int)(en >> 32); }
};
template <typename T> constexpr unsigned list_cap() { return LE<T>::CAP; }
constexpr int REG_NC = THR_NL * TW * 8 / CHUNK;   // chunks of a row kept in registers (bf16: 16)
constexpr int EBINS = 64;         // exponent bins of the top-p bound

// Keys: the value's bits with the sign bit flipped for non-negative values
// and every bit flipped for negative ones (unsigned order = value order);
// bf16 keys are the upper 16 bits of a 32-bit key, the lower ones zero.
template <typename T>
__device__ __forceinline__ uint32_t vkey(float f) {
  uint32_t u = __float_as_uint(f);
  u = (u == 0x80000000u) ? 0u : u;
  const uint32_t k = u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u);
  return sizeof(T) == 2 ? (k & 0xffff0000u) : k;
}
template <typename T>
__device__ __forceinline__ float keyv(uint32_t k) {
  const uint32_t m = (uint32_t)((int32_t)k >> 31) & 0x7fffffffu;
  const uint32_t u = ~(k ^ m);
  return __uint_as_float(sizeof(T) == 2 ? (u & 0xffff0000u) : u);
}
template <typename T> constexpr uint32_t key_neg() { return sizeof(T) == 2 ? 0x007f0000u : 0x007fffffu; }
template <typename T>
__device__ __forceinline__ uint32_t lkey(typename LE<T>::E en) {
  return vkey<T>(__uint_as_float(LE<T>::bits(en)));
}

struct ThrShared {
  union {
    unsigned c[256 * HCOPY];             // [digit][copy] counts
    unsigned long long m[256 * HCOPY];   // [digit][copy] masses (units of 2^-40)
  } h;
  union {
    uint32_t k32[LIST_BYTES / 4];
    unsigned long long k64[LIST_BYTES / 8];
  } list;                                // candidates (LE<T> entries)
  unsigned long long sink[64];           // where a lane's non-candidates are written
  uint32_t cmax[REG_NC];                 // published statistics: chunk max keys,
  unsigned long long csum[REG_NC];       // chunk masses (units of 2^-40) and
  unsigned long long csx;                // the mass of the draft id's chunk without it
  double eb[EBINS];                      // merged exponent bins
  unsigned wcnt[TNW];                    // list entries appended by each wave
  alignas(16) unsigned long long bins[256];   // merged bins of the level
  float fw[TNW];
  unsigned long long cw[TNW];
  double dw[TNW];
  double target;                         // top-p: P times the total mass
  unsigned long long above;              // count or mass above the digits chosen so far
  unsigned long long upper;              // full-row top-k: values outside digit 0
  int digit;
};

template <typename T>
__device__ __forceinline__ typename LE<T>::E* list_of(ThrShared& th) {
  if constexpr (sizeof(T) == 2) return th.list.k32;
  else return th.list.k64;
}

// round(t * 2^40) for t in [0, 1]: t * 2^40 is exact in fp32, rintf rounds it
// to nearest even (values of 2^23 and above are integers already), and the two
// 32-bit halves of the integer are exact in fp32 too
__device__ __forceinline__ unsigned long long fixmass(float t) {
  const float s = __builtin_rintf(t * 1099511627776.0f);
  const float hi = __builtin_floorf(s * 2.3283064365386963e-10f);
  const float lo = s - hi * 4294967296.0f;
  return ((unsigned long long)(uint32_t)hi << 32) | (uint32_t)lo;
}

// f(v, e) for the values of one 128-bit word of a row, in element order; e
// is the element index (e0: the word's first).
template <typename T, typename F>
__device__ __forceinline__ void each_val(const uint4& w, int e0, F& f) {
  const uint32_t d[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int h = 0; h < 4; ++h) {
    if constexpr (sizeof(T) == 4) {
      f(__uint_as_float(d[h]), e0 + h);
    } else {
      f(__uint_as_float(d[h] << 16), e0 + 2 * h);
      f(__uint_as_float(d[h] & 0xffff0000u), e0 + 2 * h + 1);
    }
  }
}

// The VEC values of a word in element order.
template <typename T>
__device__ __forceinline__ void unpack_word(const uint4& w, float* v) {
  const uint32_t d[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int h = 0; h < 4; ++h) {
    if constexpr (sizeof(T) == 4) {
      v[h] = __uint_as_float(d[h]);
    } else {
      v[2 * h] = __uint_as_float(d[h] << 16);
      v[2 * h + 1] = __uint_as_float(d[h] & 0xffff0000u);
    }
  }
}

// Word g of a row (elements [g*VEC, g*VEC + VEC)).  al: one 128-bit load from
// an offset clamped to the row's last word (thr_mask then puts -inf past
// element V); otherwise element loads with -inf past V.
template <typename T>
__device__ __forceinline__ uint4 thr_word(const T* __restrict__ rp, int g, int V, bool al) {
  constexpr int VEC = VT<T>::VEC;
  const int e0 = g * VEC;
  if (!al) return load_word_scalar<T>(rp, e0, V, NEG_INF);
  const int last = ((V - 1) / VEC) * VEC;
  return *reinterpret_cast<const uint4*>(rp + min(e0, last));
}
template <typename T>
__device__ __forceinline__ uint4 thr_mask(uint4 w, int g, int V) {
  constexpr int VEC = VT<T>::VEC;
  const int e0 = g * VEC;
  return (e0 + VEC > V) ? mask_tail<T>(w, V - e0, fill_bits<T>(NEG_INF)) : w;
}

// 64-bit DPP moves (two 32-bit moves; lanes without a source read 0), the
// wave's inclusive sum in lane order and its total, with no lane-address
// registers (a loop over the levels would keep those live across every pass)
template <int CTRL, int ROWS = 0xf>
__device__ __forceinline__ unsigned long long dpp_u64(unsigned long long x) {
  const int lo = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)x, CTRL, ROWS, 0xf, false);
  const int hi = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)(x >> 32), CTRL, ROWS, 0xf, false);
  return ((unsigned long long)(uint32_t)hi << 32) | (uint32_t)lo;
}
__device__ __forceinline__ unsigned long long wave_scan_u64(unsigned long long x) {
  x += dpp_u64<0x111>(x);         // row_shr:1
  x += dpp_u64<0x112>(x);         // row_shr:2
  x += dpp_u64<0x114>(x);         // row_shr:4
  x += dpp_u64<0x118>(x);         // row_shr:8
  x += dpp_u64<0x142, 0xa>(x);    // row_bcast:15
  x += dpp_u64<0x143, 0xc>(x);    // row_bcast:31
  return x;
}
__device__ __forceinline__ unsigned long long readlane_u64(unsigned long long x, int l) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)x, l);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(x >> 32), l);
  return ((unsigned long long)hi << 32) | lo;
}

__device__ __forceinline__ float thr_block_max(float x, ThrShared& th) {
  x = wave_reduce_rows(x, [](float a, float b) { return fmax3nan(a, b); });
  if ((threadIdx.x & 63) == 0) th.fw[threadIdx.x >> 6] = x;
  __syncthreads();
  float r = th.fw[0];
#pragma unroll
  for (int q = 1; q < TNW; ++q) r = fmax3nan(r, th.fw[q]);
  return r;
}

// Exact sum of a 64-bit count or mass over the workgroup.
__device__ __forceinline__ unsigned long long thr_block_sum(unsigned long long x, ThrShared& th) {
  x = readlane_u64(wave_scan_u64(x), 63);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) th.cw[threadIdx.x >> 6] = x;
  __syncthreads();
  unsigned long long r = 0ull;
#pragma unroll
  for (int q = 0; q < TNW; ++q) r += th.cw[q];
  return r;
}

// Sum over the workgroup in a fixed order (deterministic).
__device__ __forceinline__ double thr_block_sum_d(double x, ThrShared& th) {
  x = wave_reduce_rows(x, [](double a, double b) { return a + b; });
  __syncthreads();
  if ((threadIdx.x & 63) == 0) th.dw[threadIdx.x >> 6] = x;
  __syncthreads();
  double r = 0.0;
#pragma unroll
  for (int q = 0; q < TNW; ++q) r += th.dw[q];
  return r;
}

__device__ __forceinline__ void clear_bins(ThrShared& th) {
  uint4* hz = reinterpret_cast<uint4*>(&th.h);
  constexpr int NZ = (int)(sizeof(th.h) / 16);
  for (int i = threadIdx.x; i < NZ; i += TW) hz[i] = make_uint4(0u, 0u, 0u, 0u);
  __syncthreads();
}

// Merge the copies of each bin into th.bins (thread t: bin t/4, a quarter of
// the copies, read as 128-bit words from one base address).
template <bool MASS>
__device__ __forceinline__ void merge_bins(ThrShared& th) {
  static_assert(HCOPY == 32, "a quarter of the copies is eight words");
  const int tid = threadIdx.x;
  const int d = tid >> 2, part = tid & 3;
  unsigned long long s = 0ull;
  if constexpr (MASS) {
    const ulonglong2* p = reinterpret_cast<const ulonglong2*>(&th.h.m[d * HCOPY + part * 8]);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const ulonglong2 v = p[q];
      s += v.x + v.y;
    }
  } else {
    const uint4* p = reinterpret_cast<const uint4*>(&th.h.c[d * HCOPY + part * 8]);
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const uint4 v = p[q];
      s += (unsigned long long)v.x + v.y + v.z + v.w;
    }
  }
  s += dpp_u64<DPP_XOR1>(s);
  s += dpp_u64<DPP_XOR2>(s);
  if (part == 0) th.bins[d] = s;
  __syncthreads();
}

// Wave 0 picks the highest digit whose bins from the top, with everything
// above from earlier levels, reach the goal: K values (counts) or the target
// mass (masses).  At level 0 the target is P times z, or times the level's
// total when z < 0.
template <bool MASS>
__device__ __forceinline__ void pick_digit(ThrShared& th, int lev, unsigned K, float Pp,
                                           double z = -1.0) {
  const int tid = threadIdx.x;
  if (tid < 64) {
    const int l = tid;
    // this lane's digits 255 - 4l down to 252 - 4l
    const ulonglong2* bp = reinterpret_cast<const ulonglong2*>(&th.bins[252 - 4 * l]);
    const ulonglong2 b01 = bp[0], b23 = bp[1];
    const unsigned long long bb[4] = {b23.y, b23.x, b01.y, b01.x};
    const unsigned long long ls = bb[0] + bb[1] + bb[2] + bb[3];
    const unsigned long long inc = wave_scan_u64(ls);
    const unsigned long long total = readlane_u64(inc, 63);
    const unsigned long long base = lev == 0 ? 0ull : th.above;
    const double tgt = lev == 0 ? (double)Pp * (z < 0.0 ? (double)total : z) : th.target;
    unsigned long long c = base + inc - ls;
    int first = 4;
    unsigned long long at = 0ull;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const unsigned long long ci = c + bb[i];
      const bool hit = MASS ? ((double)ci >= tgt) : (ci >= (unsigned long long)K);
      if (first == 4 && hit) {
        first = i;
        at = c;
      }
      c = ci;
    }
    const uint64_t msk = __ballot(first < 4);
    const int src = msk ? (int)__builtin_ctzll(msk) : 0;
    const int f = __builtin_amdgcn_readlane(first, src);
    const unsigned long long ab = readlane_u64(at, src);
    if (l == 0) {
      th.digit = msk ? 255 - (4 * src + f) : 0;
      th.above = msk ? ab : base;
      if (lev == 0) th.target = tgt;
    }
  }
  __syncthreads();
}

// Radix select over the keys of the list: the K-th largest key (MASS false),
// or the key of the top-p cut of the keys at or above kfloor (MASS true; z the
// total mass of the set the cut is taken in, or < 0 for the listed keys').
// A list of at most LIST_SMALL entries adds straight into the merged bins
// (one copy: few atomics meet on one address), a longer one into the copies.
constexpr unsigned LIST_SMALL = 2048;
template <typename T, bool MASS>
__device__ __forceinline__ uint32_t list_select(ThrShared& th, unsigned n, unsigned K, float Pp,
                                                double z, uint32_t kfloor, float M, float c) {
  constexpr int LEVELS = sizeof(T) == 2 ? 2 : 4;
  const int cp = threadIdx.x & (HCOPY - 1);
  const bool small = n <= LIST_SMALL;
  const typename LE<T>::E* lst = list_of<T>(th);
  uint32_t prefix = 0u, pmask = 0u;
#pragma unroll
  for (int lev = 0; lev < LEVELS; ++lev) {
    const int shift = 24 - 8 * lev;
    if (small) {
      if (threadIdx.x < 256) th.bins[threadIdx.x] = 0ull;
      __syncthreads();
    } else {
      clear_bins(th);
    }
    // each wave walks its own segment of the list
    const int wv = threadIdx.x >> 6;
    const unsigned seg = list_cap<T>() / TNW;
    const unsigned nw = th.wcnt[wv];
    for (unsigned i = (threadIdx.x & 63); i < nw; i += 64) {
      const uint32_t k = lkey<T>(lst[wv * seg + i]);
      if (k >= kfloor && (k & pmask) == prefix) {
        const uint32_t d = (k >> shift) & 255u;
        if constexpr (MASS) {
          const unsigned long long f = fixmass(term(keyv<T>(k), M, c));
          if (small) atomicAdd(&th.bins[d], f);
          else atomicAdd(&th.h.m[d * HCOPY + cp], f);
        } else {
          if (small) atomicAdd(&th.bins[d], 1ull);
          else atomicAdd(&th.h.c[d * HCOPY + cp], 1u);
        }
      }
    }
    __syncthreads();
    if (!small) merge_bins<MASS>(th);
    pick_digit<MASS>(th, lev, K, Pp, z);
    prefix |= (uint32_t)th.digit << shift;
    pmask |= 255u << shift;
  }
  return prefix;
}

// Statistics of a row whose kept values are all on the list (keys >= tkey):
// per chunk the max and the sum of exp2((v - m_c) c) under the threshold, as
// the producers of k_verify publish them (one self-tagged word per chunk at
// stat), and for the chunk that holds the draft id x the same sum without x
// (prefix-match requests: of the values before x) at sxw.  Maxima by an
// integer max over the keys; masses as integers in units of 2^-40, so the
// sums do not depend on the order of the atomics.  A wave's segment is in
// element order, so 64 consecutive entries mostly share a chunk: such a
// window is reduced across the wave first and takes one atomic.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t x) {
  x = max(x, (uint32_t)dpp_i<DPP_XOR1>((int)x));
  x = max(x, (uint32_t)dpp_i<DPP_XOR2>((int)x));
  x = max(x, (uint32_t)dpp_i<DPP_HMIRROR>((int)x));
  x = max(x, (uint32_t)dpp_i<DPP_MIRROR>((int)x));
  return max(max((uint32_t)__builtin_amdgcn_readlane((int)x, 0), (uint32_t)__builtin_amdgcn_readlane((int)x, 16)),
             max((uint32_t)__builtin_amdgcn_readlane((int)x, 32), (uint32_t)__builtin_amdgcn_readlane((int)x, 48)));
}

template <typename T>
__device__ __forceinline__ void publish_stats(ThrShared& th, uint32_t tkey, float c, int nc, int x,
                                              bool match, u64* stat, u64* sxw) {
  const int tid = threadIdx.x;
  const int wv = tid >> 6;
  const int lane = tid & 63;
  const unsigned seg = list_cap<T>() / TNW;
  const unsigned nw = th.wcnt[wv];
  if (tid < REG_NC) {
    th.cmax[tid] = 0u;
    th.csum[tid] = 0ull;
  }
  if (tid == 0) th.csx = 0ull;
  __syncthreads();
  const typename LE<T>::E* lst = list_of<T>(th) + wv * seg;
  // the window's chunk when all its kept entries share one (-1: none kept,
  // -2: several)
  auto window_chunk = [&](int cc) -> int {
    const uint64_t live = __ballot(cc >= 0);
    if (!live) return -1;
    const int c0 = __builtin_amdgcn_readlane(cc, (int)__builtin_ctzll(live));
    return __ballot(cc >= 0 && cc != c0) ? -2 : c0;
  };
  for (unsigned b0 = 0; b0 < nw; b0 += 64) {
    const unsigned i = b0 + lane;
    uint32_t k = 0u;
    int cc = -1;
    if (i < nw) {
      const typename LE<T>::E en = lst[i];
      const uint32_t kk = lkey<T>(en);
      if (kk >= tkey) {
        k = kk;
        cc = LE<T>::index(en, wv) / CHUNK;
      }
    }
    const int wc = window_chunk(cc);
    if (wc >= 0) {
      const uint32_t km = wave_max_u32(k);
      if (lane == 0) atomicMax(&th.cmax[wc], km);
    } else if (wc == -2 && cc >= 0) {
      atomicMax(&th.cmax[cc], k);
    }
  }
  __syncthreads();
  const int xc = x >= 0 ? x / CHUNK : -1;
  for (unsigned b0 = 0; b0 < nw; b0 += 64) {
    const unsigned i = b0 + lane;
    unsigned long long fx = 0ull, fs = 0ull;
    int cc = -1;
    if (i < nw) {
      const typename LE<T>::E en = lst[i];
      const uint32_t k = lkey<T>(en);
      if (k >= tkey) {
        const int e = LE<T>::index(en, wv);
        cc = e / CHUNK;
        fx = fixmass(term(keyv<T>(k), keyv<T>(th.cmax[cc]), c));
        if (cc == xc && (match ? e < x : e != x)) fs = fx;
      }
    }
    const int wc = window_chunk(cc);
    if (wc >= 0) {
      const unsigned long long sw = readlane_u64(wave_scan_u64(fx), 63);
      const unsigned long long sx = wc == xc ? readlane_u64(wave_scan_u64(fs), 63) : 0ull;
      if (lane == 0) {
        atomicAdd(&th.csum[wc], sw);
        if (sx) atomicAdd(&th.csx, sx);
      }
    } else if (wc == -2 && cc >= 0) {
      atomicAdd(&th.csum[cc], fx);
      if (fs) atomicAdd(&th.csx, fs);
    }
  }
  __syncthreads();
  constexpr double UNIT = 9.094947017729282e-13;   // 2^-40
  if (tid < nc) {
    const uint32_t mk = th.cmax[tid];   // no finite value has key 0
    const float m = mk ? keyv<T>(mk) : NEG_INF;
    const float sm = mk ? (float)((double)th.csum[tid] * UNIT) : 0.f;
    put_w(stat + tid, __float_as_uint(sm) & ~TAG, __float_as_uint(m));
  }
  if (tid == 0 && sxw != nullptr && x >= 0)
    put_w(sxw, 0u, __float_as_uint((float)((double)th.csx * UNIT)));
}

// The row's threshold in tau.  The variant that keeps the row in registers
// (REG) returns false, with nothing written, where a full-row fallback is
// needed; the caller then runs the variant that reads the row for each pass.
// With stat != nullptr the register variant also publishes the row's
// statistics (publish_stats) whenever its threshold came from a list, and
// sets published.
template <typename T, bool REG>
__device__ __forceinline__ bool row_threshold(const T* __restrict__ rp, int V, bool al,
                                              const Req& R, ThrShared& th, float& tau,
                                              u64* stat = nullptr, int x = -1,
                                              u64* sxw = nullptr, bool* published = nullptr) {
  constexpr int VEC = VT<T>::VEC;
  constexpr int LEVELS = sizeof(T) == 2 ? 2 : 4;
  constexpr uint32_t KNEG = key_neg<T>();
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int cp = tid & (HCOPY - 1);
  uint4 w[REG ? THR_NL : 1];
  if constexpr (REG) {
    // word i of every thread covers elements [i*TW*VEC, (i+1)*TW*VEC): only the
    // one that holds the row's end needs per-lane clamps and masks (the
    // conditions are uniform)
    const T* base = rp + tid * VEC;
    const uint32_t nb = fill_bits<T>(NEG_INF);
    const uint32_t nw = sizeof(T) == 4 ? nb : (nb | (nb << 16));
#pragma unroll
    for (int i = 0; i < THR_NL; ++i) {
      const int g0 = i * TW * VEC;
      if (g0 + TW * VEC <= V) w[i] = *reinterpret_cast<const uint4*>(base + g0);
      else if (g0 < V) w[i] = thr_mask<T>(thr_word<T>(rp, i * TW + tid, V, true), i * TW + tid, V);
      else w[i] = make_uint4(nw, nw, nw, nw);
    }
  }
  // each_read_w(f): f(word, e0) for every word of the thread (e0 the index of
  // the word's first value), read from the row eight words at a time.  The
  // trip count is the same in every lane (f may use wave-wide operations):
  // words past the row's end, and values past element V, read as -inf
  auto each_read_w = [&](auto&& f) {
    const int ng = (V + VEC - 1) / VEC;
    for (int base = 0; base < ng; base += 8 * TW) {
      const int g0 = base + tid;
      uint4 q[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) q[i] = thr_word<T>(rp, min(g0 + i * TW, ng - 1), V, al);
#pragma unroll
      for (int i = 0; i < 8; ++i) f(thr_mask<T>(q[i], g0 + i * TW, V), (g0 + i * TW) * VEC);
    }
  };
  // each_w(f): the same from the registers when the row is kept there
  auto each_w = [&](auto&& f) {
    if constexpr (REG) {
      // the words pass through an empty asm statement first: what a pass
      // derives from them does not depend on the level, and the compiler
      // would otherwise keep it for every value across the levels
#pragma unroll
      for (int i = 0; i < THR_NL; ++i)
        asm volatile("" : "+v"(w[i].x), "+v"(w[i].y), "+v"(w[i].z), "+v"(w[i].w));
#pragma unroll
      for (int i = 0; i < THR_NL; ++i) f(w[i], (i * TW + tid) * VEC);
    } else {
      each_read_w(f);
    }
  };
  // each(f) / each_read(f): f(v, e) for every value
  auto each = [&](auto&& f) { each_w([&](const uint4& x, int e0) { each_val<T>(x, e0, f); }); };
  auto each_read = [&](auto&& f) {
    each_read_w([&](const uint4& x, int e0) { each_val<T>(x, e0, f); });
  };
  // fill_list(vlo): every value at or above vlo goes to the list, each wave's
  // to its own segment, word by word (a word's values at consecutive places
  // from the lane's offset in the wave's prefix sum of the counts); the
  // wave's count stays in a register.  Returns the number of entries, or a
  // number above the capacity when a segment overflowed.
  constexpr unsigned SEG = list_cap<T>() / TNW;
  auto fill_list = [&](float vlo) -> unsigned {
    using E = typename LE<T>::E;
    E* lst = list_of<T>(th) + (unsigned)(tid >> 6) * SEG;
    E* sink = reinterpret_cast<E*>(&th.sink[lane]);
    unsigned wc = 0u;
    each_w([&](const uint4& x, int e0) {
      float v[VEC];
      unpack_word<T>(x, v);
      float wm = v[0];
#pragma unroll
      for (int h = 1; h < VEC; ++h) wm = __builtin_fmaxf(wm, v[h]);
      if (__ballot(wm >= vlo)) {
        int cnt = 0;
#pragma unroll
        for (int h = 0; h < VEC; ++h) cnt += v[h] >= vlo ? 1 : 0;
        const int inc = wave_scan_add(cnt);
        const unsigned tot = (unsigned)__builtin_amdgcn_readlane(inc, 63);
        if (wc + tot <= SEG) {
          // every value is written, a candidate to its place and the rest to
          // the lane's sink slot (no branch per value)
          unsigned pos = wc + (unsigned)(inc - cnt);
#pragma unroll
          for (int h = 0; h < VEC; ++h) {
            const bool hit = v[h] >= vlo;
            E* at = hit ? lst + pos : sink;
            *at = LE<T>::make(__float_as_uint(v[h] + 0.f), e0 + h);
            pos += hit ? 1u : 0u;
          }
        }
        wc += tot;
      }
    });
    if (lane == 0) th.wcnt[tid >> 6] = wc;
    __syncthreads();
    unsigned n = 0u, big = 0u;
#pragma unroll
    for (int q = 0; q < TNW; ++q) {
      n += th.wcnt[q];
      big = max(big, th.wcnt[q]);
    }
    return big > SEG ? list_cap<T>() + 1u : n;
  };

  // row max and each thread's own max, NaN-propagating: a row that holds a
  // NaN or +inf, or only -inf, is left unfiltered and unpublished, and the
  // row pass of the verify kernel reports it
  float tmax = NEG_INF;
  {
    float mh = NEG_INF, ml = NEG_INF;
    auto wmax = [&](const uint4& q) {
      const uint32_t d[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        if constexpr (sizeof(T) == 2) {
          mh = fmax3nan(mh, __uint_as_float(d[h] & 0xffff0000u));
          ml = fmax3nan(ml, __uint_as_float(d[h] << 16));
        } else {
          mh = fmax3nan(mh, __uint_as_float(d[h]));
        }
      }
    };
    if constexpr (REG) {
#pragma unroll
      for (int i = 0; i < THR_NL; ++i) wmax(w[i]);
    } else {
      const int ng = (V + VEC - 1) / VEC;
      for (int g = tid; g < ng; g += TW) wmax(thr_mask<T>(thr_word<T>(rp, g, V, al), g, V));
    }
    tmax = fmax3nan(mh, ml);
  }
  const float M = thr_block_max(tmax, th);
  tau = NEG_INF;
  if (!(M > NEG_INF && M < POS_INF)) return true;

  bool do_k = R.K > 0;
  const bool do_p = R.P > 0.f && R.P < 1.f;
  uint32_t tau_key = 0u;   // keep everything
  unsigned n_list = 0u;    // valid list entries (0: no list)
  if (do_k) {
    const unsigned K = (unsigned)R.K;
    bool full = true;      // full-row passes
    if (K <= (unsigned)TW) {
      // a lower bound of the K-th largest value: each wave finds the r-th
      // largest of its threads' maxima, r = ceil(K / 16), by a binary search
      // over the key bits with ballot counts; r values of the wave are at or
      // above it, so K values are at or above the smallest of the 16
      const unsigned r = (K + TNW - 1) / TNW;
      const uint32_t kt = vkey<T>(tmax);
      uint32_t t = 0u;
#pragma unroll
      for (int bit = 31; bit >= (sizeof(T) == 2 ? 16 : 0); --bit) {
        const uint32_t cand = t | (1u << bit);
        if ((unsigned)__popcll(__ballot(kt >= cand)) >= r) t = cand;
      }
      if (lane == 0) th.cw[tid >> 6] = t;
      __syncthreads();
      uint32_t lbk = 0xffffffffu;
#pragma unroll
      for (int q = 0; q < TNW; ++q) lbk = min(lbk, (uint32_t)th.cw[q]);
      const float lb = keyv<T>(lbk);
      if (lb > NEG_INF) {
        const unsigned n = fill_list(lb);
        if (n <= list_cap<T>()) {
          full = false;
          bool keep_all = false;
          if (n == K) {
            // exactly K candidates: K is below the number of finite values
            // only if a finite value lies below the bound
            unsigned long long below = 0ull;
            each([&](float v, int) { below += (v > NEG_INF && v < lb) ? 1ull : 0ull; });
            keep_all = thr_block_sum(below, th) == 0ull;
          }
          if (keep_all) {
            do_k = false;
          } else {
            tau_key = list_select<T, false>(th, n, K, 0.f, -1.0, 0u, M, R.c);
            n_list = n;
          }
        }
      }
    }
    if constexpr (REG) {
      if (full) return false;
    } else if (full) {
      uint32_t prefix = 0u, pmask = 0u;
      unsigned long long ninf = 0ull;   // -inf values and padding (counted only when needed)
#pragma unroll
      for (int lev = 0; lev < LEVELS; ++lev) {
        const int shift = 24 - 8 * lev;
        clear_bins(th);
        // -inf and the padding land in digit 0 at level 0
        each_read([&](float v, int) {
          const uint32_t k = vkey<T>(v);
          if ((k & pmask) == prefix) atomicAdd(&th.h.c[((k >> shift) & 255u) * HCOPY + cp], 1u);
        });
        __syncthreads();
        merge_bins<false>(th);
        if (lev == 0) {
          // count -inf only if the select can reach digit 0 or K may not be
          // below the number of finite values
          if (tid < 64) {
            const ulonglong2* bp = reinterpret_cast<const ulonglong2*>(&th.bins[4 * tid]);
            const ulonglong2 b01 = bp[0], b23 = bp[1];
            const unsigned long long u = (tid ? b01.x : 0ull) + b01.y + b23.x + b23.y;
            const unsigned long long tot = readlane_u64(wave_scan_u64(u), 63);
            if (tid == 0) th.upper = tot;
          }
          __syncthreads();
          if (th.upper <= (unsigned long long)K) {
            unsigned long long n = 0ull;
            each_read([&](float v, int) { n += (v == NEG_INF) ? 1ull : 0ull; });
            ninf = thr_block_sum(n, th);
            if ((unsigned long long)K >= th.upper + th.bins[0] - ninf) {
              do_k = false;
              break;
            }
          }
        }
        // -inf values still inside the prefix are not candidates
        if (tid == 0 && ninf != 0ull && (KNEG & pmask) == prefix) th.bins[(KNEG >> shift) & 255u] -= ninf;
        __syncthreads();
        pick_digit<false>(th, lev, K, 0.f);
        prefix |= (uint32_t)th.digit << shift;
        pmask |= 255u << shift;
      }
      if (do_k) tau_key = prefix;
    }
  }
  if (do_p) {
    uint32_t pk = 0u;
    bool full = true;
    if (do_k && n_list != 0u) {
      // the top-k set is on the list
      pk = list_select<T, true>(th, n_list, 0u, R.P, -1.0, tau_key, M, R.c);
      full = false;
    } else if (!do_k) {
      // the total mass, exact, and the terms by binary exponent: bin b holds
      // the terms in [2^-b, 2^(1-b)), the last bin everything below
      clear_bins(th);
      double zs = 0.0;
      float zw = 0.f;
      int nz = 0;
      each([&](float v, int) {
        const float t = term(v, M, R.c);
        zw += t;
        if (++nz == VEC) {   // a word's values (a compile-time count when unrolled)
          zs += (double)zw;
          zw = 0.f;
          nz = 0;
        }
        // t = (q + f) 2^-(b+12) with 4,096 <= q < 8,192 and 0 <= f < 1 for
        // b < 63; the last bin's terms are all below 2^-62
        const uint32_t tb = __float_as_uint(t);
        const uint32_t b = min(127u - (tb >> 23), (uint32_t)(EBINS - 1));
        atomicAdd(&th.h.c[b * HCOPY + cp], 0x1000u | ((tb >> 11) & 0xfffu));
      });
      zs += (double)zw;
      const double Zs = thr_block_sum_d(zs, th);
      const unsigned long long Z = (unsigned long long)(Zs * 1099511627776.0);
      if (tid < EBINS) {
        unsigned long long sq = 0ull;
#pragma unroll
        for (int q = 0; q < HCOPY; ++q) sq += th.h.c[tid * HCOPY + q];
        // within 2^-12 below the bin's sum; the last bin is bounded by count
        th.eb[tid] = tid < EBINS - 1 ? ldexp((double)sq, -(tid + 12)) : ldexp((double)V, -62);
      }
      __syncthreads();
      // the first exponent whose tail below is light enough (the tails shrink
      // as the exponent grows, and the last one is empty)
      if (tid < 64) {
        double tail = 0.0;
        for (int b = tid + 1; b < EBINS; ++b) tail += th.eb[b];
        const bool light = 1.01 * tail * 1099511627776.0 < (1.0 - (double)R.P) * (double)Z;
        const uint64_t msk = __ballot(tid < EBINS && light);
        if (tid == 0) th.digit = msk ? (int)__builtin_ctzll(msk) : EBINS - 1;
      }
      __syncthreads();
      // every value whose term reaches 2^-bc is at or above vlo (a factor 2
      // of margin in the term for the rounding of (v - M) c and of exp2)
      const int bc = th.digit;
      const float vlo = __double2float_rd((double)M - (double)(bc + 1) / (double)R.c);
      if (bc < EBINS - 1 && vlo > NEG_INF) {
        const unsigned n = fill_list(vlo);
        if (n <= list_cap<T>()) {
          pk = list_select<T, true>(th, n, 0u, R.P, (double)Z, 0u, M, R.c);
          full = false;
        }
      }
    }
    if constexpr (REG) {
      if (full) return false;
    } else if (full) {
      // the top-k set, -inf excluded (its masses are 0 anyway)
      const uint32_t kfloor = do_k ? tau_key : KNEG + 1u;
      uint32_t prefix = 0u, pmask = 0u;
#pragma unroll
      for (int lev = 0; lev < LEVELS; ++lev) {
        const int shift = 24 - 8 * lev;
        clear_bins(th);
        each_read([&](float v, int) {
          const uint32_t k = vkey<T>(v);
          if (k >= kfloor && (k & pmask) == prefix)
            atomicAdd(&th.h.m[((k >> shift) & 255u) * HCOPY + cp], fixmass(term(v, M, R.c)));
        });
        __syncthreads();
        merge_bins<true>(th);
        pick_digit<true>(th, lev, 0u, R.P);
        prefix |= (uint32_t)th.digit << shift;
        pmask |= 255u << shift;
      }
      pk = prefix;
    }
    tau_key = pk > tau_key ? pk : tau_key;
  }
  tau = (do_k || do_p) ? keyv<T>(tau_key) : NEG_INF;
  if constexpr (REG) {
    // every selection of this variant ran on the list, so the kept values
    // (keys >= tau_key) are all on it
    if (stat != nullptr && (do_k || do_p)) {
      publish_stats<T>(th, tau_key, R.c, (V + CHUNK - 1) / CHUNK, x, R.kind == SV_DRAFT_MATCH,
                       stat, sxw);
      *published = true;
    }
  }
  return true;
}

template <typename T>
__device__ __forceinline__ float thr_row(const T* __restrict__ rp, int64_t ld, int V, const Req& R,
                                         ThrShared& th, u64* stat, int x, u64* sxw,
                                         bool& published) {
  const bool al = (((uintptr_t)rp & 15) == 0) && (((ld * (int64_t)sizeof(T)) & 15) == 0);
  float tau = NEG_INF;
  published = false;
  if (al && V <= THR_NL * TW * VT<T>::VEC &&
      row_threshold<T, true>(rp, V, true, R, th, tau, stat, x, sxw, &published))
    return tau;
  __syncthreads();   // the register variant's last LDS reads are done
  row_threshold<T, false>(rp, V, al, R, th, tau);
  return tau;
}

template <typename TT, typename TD, int E>
__global__ __launch_bounds__(TW) void k_thresh(const Params P) {
  __shared__ ThrShared th;
  int bid = blockIdx.x;
  const int side = bid & 1;   // 0 target row, 1 draft row
  bid >>= 1;
  const int j = bid % (P.max_k + 1);
  const int b = bid / (P.max_k + 1);
  // scalar loads decide which workgroups have a row; only those check the
  // offsets the way k_verify does (rows of an invalid request may be another's)
  const int cu0 = ldu(P.cu + b);
  const int cu1 = ldu(P.cu + b + 1);
  const int k = cu1 - cu0 - 1;
  const Req R = load_req(P, b);
  if (j > k || R.greedy || R.bad_param || !R.filt) return;
  if (side == 1 && (R.kind != SV_DRAFT_LOGITS || j >= k)) return;
  if (!offsets_ok<E>(P, b, cu0, cu1)) return;
  const int d0 = cu0 - b;
  u64* out = side == 0 ? P.thr_t + cu0 + j : P.thr_d + (d0 + j);
  // the statistics words of the row, and for a target row with a draft id in
  // range the words of the values at it
  u64* stat = side == 0 ? P.cst + (int64_t)(cu0 + j) * P.nc : P.dst + (int64_t)(d0 + j) * P.nc;
  const int xr = (side == 0 && j < k) ? ldu(P.drafts + d0 + j) : -1;
  const int x = (xr >= 0 && xr < P.vocab) ? xr : -1;
  u64* rx = P.rx + (int64_t)(cu0 + j) * 3;
  const TT* trow = target_rows<TT>(P, R.pen) + (int64_t)(cu0 + j) * P.ld_t;
  const TD* drow = (const TD*)P.draft + (int64_t)(d0 + j) * P.ld_d;
  float tau;
  bool pub;
  if constexpr (std::is_same<TT, TD>::value) {   // one copy of the code for both sides
    tau = thr_row<TT>(side == 0 ? trow : drow, side == 0 ? P.ld_t : P.ld_d, P.vocab, R, th, stat,
                      x, x >= 0 ? rx + 1 : nullptr, pub);
  } else if (side == 0) {
    tau = thr_row<TT>(trow, P.ld_t, P.vocab, R, th, stat, x, x >= 0 ? rx + 1 : nullptr, pub);
  } else {
    tau = thr_row<TD>(drow, P.ld_d, P.vocab, R, th, stat, -1, nullptr, pub);
  }
  if (threadIdx.x == 0) {
    if (pub && x >= 0) {
      float lx = to_f(trow[x]);
      if (lx < tau) lx = NEG_INF;
      put_w(rx + 0, 0u, __float_as_uint(lx));
      if (R.kind == SV_DRAFT_LOGITS || R.kind == SV_DRAFT_PROBS)
        put_w(rx + 2, 0u, __float_as_uint(to_f(drow[x])));
    }
    *out = ((u64)(pub ? THR_PUBLISHED : 0u) << 32) | (u64)__float_as_uint(tau);
  }
}

// ---------------------------------------------------------------------------
// k_penalize: presence / frequency penalties (the penalized entry point)
// ---------------------------------------------------------------------------
// One workgroup per verify row j of a request with a nonzero penalty: the row
// is copied to the same place in P.pen, then every token t the row counts
// as generated (c(t) = history count + occurrences among the drafts x_0 ..
// x_{j-1}, c > 0) gets l(t) - (frequency c + presence), evaluated in fp64 and
// rounded to fp32, then to the logits' type (nearest, ties to even).  Each
// such token is written once: a history entry counts the drafts equal to its
// token and marks them; a draft not marked is written by its first occurrence.
__device__ __forceinline__ void store_pen(float* row, int t, double v) {
  row[t] = __double2float_rn(v);
}
__device__ __forceinline__ void store_pen(uint16_t* row, int t, double v) {
  const float f = __double2float_rn(v);
  uint32_t u = __float_as_uint(f);
  u = (f != f) ? 0x7fc00000u : u + 0x7fffu + ((u >> 16) & 1u);
  row[t] = (uint16_t)(u >> 16);
}

template <typename TT, int E>
__global__ __launch_bounds__(WG) void k_penalize(const Params P) {
  __shared__ int xs[MAX_K + 1];
  __shared__ int marked[MAX_K + 1];
  const int tid = threadIdx.x;
  const int j = blockIdx.x % (P.max_k + 1);
  const int b = blockIdx.x / (P.max_k + 1);
  const int cu0 = ldu(P.cu + b), cu1 = ldu(P.cu + b + 1);
  const int k = cu1 - cu0 - 1;
  const float ap = ldu(P.pres + b), af = ldu(P.freq + b);
  if (j > k || !(ap != 0.f || af != 0.f) || !(__builtin_isfinite(ap) && __builtin_isfinite(af)))
    return;
  if (!offsets_ok<E>(P, b, cu0, cu1)) return;   // the verdict k_verify gives
  const int V = P.vocab;
  const int row = cu0 + j;
  const TT* src = (const TT*)P.target + (int64_t)row * P.ld_t;
  TT* dst = (TT*)const_cast<void*>(P.pen) + (int64_t)row * P.ld_t;
  constexpr int VEC = VT<TT>::VEC;
  const bool al = ((((uintptr_t)src) | ((uintptr_t)dst)) & 15) == 0;
  int e = 0;
  if (al) {
    for (e = tid * VEC; e + VEC <= V; e += WG * VEC)
      *reinterpret_cast<uint4*>(dst + e) = *reinterpret_cast<const uint4*>(src + e);
    e = (V / VEC) * VEC + tid;
  } else {
    e = tid;
  }
  for (; e < V; e += WG) dst[e] = src[e];
  const int d0 = cu0 - b;
  if (tid < j) {
    xs[tid] = P.drafts[d0 + tid];
    marked[tid] = 0;
  }
  __syncthreads();   // the copy's stores land before the updates below
  const double fa = (double)af, pa = (double)ap;
  int h0 = P.hist_off ? P.hist_off[b] : 0, h1 = P.hist_off ? P.hist_off[b + 1] : 0;
  if (!(0 <= h0 && h0 <= h1 && (int64_t)h1 <= P.hist_nnz)) h0 = h1 = 0;
  for (int h = h0 + tid; h < h1; h += WG) {
    const int t = P.hist_tok[h];
    const int n = P.hist_cnt[h];
    if (t < 0 || t >= V || n < 0) continue;
    int c = n;
    for (int i = 0; i < j; ++i) {
      if (xs[i] == t) {
        ++c;
        marked[i] = 1;
      }
    }
    if (c > 0) store_pen(dst, t, (double)to_f(src[t]) - (fa * (double)c + pa));
  }
  __syncthreads();
  if (tid < j) {
    const int t = xs[tid];
    bool first = t >= 0 && t < V && !marked[tid];
    for (int i = 0; i < tid; ++i) first = first && xs[i] != t;
    if (first) {
      int c = 0;
      for (int i = 0; i < j; ++i) c += xs[i] == t ? 1 : 0;
      store_pen(dst, t, (double)to_f(src[t]) - (fa * (double)c + pa));
    }
  }
}

__global__ void k_fill_zero(uint4* p, size_t n16, unsigned char* tail, size_t ntail) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t q = i; q < n16; q += stride) p[q] = make_uint4(0u, 0u, 0u, 0u);
  if (i < ntail) tail[i] = 0;
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
struct Layout {
  size_t cst, dst, rx, dec, res, thr_t, thr_d, pq, ctl, order, okb, total;
};

static size_t align_up(size_t x) { return (x + 255) & ~(size_t)255; }

static bool layout(int batch, int total_rows, int vocab, int max_k, Layout& L, int& nc) {
  if (batch < 1 || total_rows < batch || vocab < 1 || max_k < 0 || max_k > MAX_K) return false;
  nc = (vocab + CHUNK - 1) / CHUNK;
  if (nc > MAX_NC) return false;
  if ((size_t)8 * (2 * max_k + 1) * nc > (size_t)STAGE_MAX) return false;
  const size_t B = (size_t)batch, R = (size_t)total_rows, D = (size_t)(total_rows - batch);
  const size_t D1 = D ? D : 1;
  size_t o = 0;
  // the control words sit at a fixed place whatever the sizes: a workspace
  // serves calls of any size, and the other regions move with them
  L.ctl = o; o = align_up(o + 32 * sizeof(u64));
  L.cst = o; o = align_up(o + R * nc * sizeof(u64));
  L.dst = o; o = align_up(o + D1 * nc * sizeof(u64));
  L.rx = o; o = align_up(o + R * 3 * sizeof(u64));
  L.dec = o; o = align_up(o + B * nc * DEC_W * sizeof(u64));
  L.res = o; o = align_up(o + B * nc * (nc <= PEER_MAX ? nc : 1) * sizeof(u64));
  L.thr_t = o; o = align_up(o + R * sizeof(u64));
  L.thr_d = o; o = align_up(o + D1 * sizeof(u64));
  L.pq = o; o = align_up(o + B * (size_t)(2 * max_k + 1) * sizeof(u64));
  L.order = o; o = align_up(o + B * 4 * sizeof(int32_t));
  L.okb = o; o = align_up(o + B * sizeof(int32_t));
  L.total = o;
  return true;
}

template <typename TT>
static long long verify_grid(const Params& P) {
  return (long long)P.batch * (P.max_k + 1) * P.ns + (long long)P.batch * P.H +
         (P.dsplit ? (long long)P.batch * P.max_k * P.ns : 0);
}

template <typename TT, typename TD>
static int launch_all(Params P, bool sampled, bool filters, bool aligned, hipStream_t st) {
  P.S = Strip<TT>::S;   // at most 8: a strip's statistics fit ProdShared::pub
  P.ns = (P.nc + P.S - 1) / P.S;
  P.H = sampled ? P.nc : 0;
  P.dsplit = (sampled && P.draft != nullptr) ? 1 : 0;
  const long long g = verify_grid<TT>(P);
  if (g >= (1LL << 31)) return SV_ERR_SHAPE;
  const size_t lds = (size_t)8 * (2 * P.max_k + 1) * P.nc;
  if (P.batch > 64) {
    hipLaunchKernelGGL(k_order, dim3(1), dim3(1024), 0, st, P);
  } else {
    P.order = nullptr;
    P.okb = nullptr;
  }
  // requests per lane when finding a request by launch position or checking
  // its offsets
  if (P.pen) {
    const long long gp = (long long)P.batch * (P.max_k + 1);
    if (P.batch <= 64)
      hipLaunchKernelGGL((k_penalize<TT, 1>), dim3((unsigned)gp), dim3(WG), 0, st, P);
    else
      hipLaunchKernelGGL((k_penalize<TT, 16>), dim3((unsigned)gp), dim3(WG), 0, st, P);
  }
  if (filters) {
    const long long g0 = (long long)P.batch * (P.max_k + 1) * 2;
    if (P.batch <= 64)
      hipLaunchKernelGGL((k_thresh<TT, TD, 1>), dim3((unsigned)g0), dim3(TW), 0, st, P);
    else
      hipLaunchKernelGGL((k_thresh<TT, TD, 16>), dim3((unsigned)g0), dim3(TW), 0, st, P);
  }
  if (P.batch <= 64) {
    if (aligned)
      hipLaunchKernelGGL((k_verify<TT, TD, true, 1>), dim3((unsigned)g), dim3(WG), lds, st, P);
    else
      hipLaunchKernelGGL((k_verify<TT, TD, false, 1>), dim3((unsigned)g), dim3(WG), lds, st, P);
  } else {
    if (aligned)
      hipLaunchKernelGGL((k_verify<TT, TD, true, 16>), dim3((unsigned)g), dim3(WG), lds, st, P);
    else
      hipLaunchKernelGGL((k_verify<TT, TD, false, 16>), dim3((unsigned)g), dim3(WG), lds, st, P);
  }
  return hipGetLastError() == hipSuccess ? SV_OK : SV_ERR_LAUNCH;
}

// Rows take 128-bit loads when the buffer's base address and row pitch are
// multiples of 16 bytes.
static bool rows_aligned(const void* base, int64_t ld, int elem) {
  return base == nullptr || (((uintptr_t)base & 15) == 0 && ((ld * elem) & 15) == 0);
}

static int dispatch(const Params& P, int tdt, int ddt, bool sampled, bool filters,
                    hipStream_t st) {
  const bool al = rows_aligned(P.target, P.ld_t, tdt == SV_F32 ? 4 : 2) &&
                  rows_aligned(P.pen, P.ld_t, tdt == SV_F32 ? 4 : 2) &&
                  rows_aligned(P.draft, P.ld_d, ddt == SV_F32 ? 4 : 2);
  if (tdt == SV_F32 && ddt == SV_F32)
    return launch_all<float, float>(P, sampled, filters, al, st);
  if (tdt == SV_F32 && ddt == SV_BF16)
    return launch_all<float, uint16_t>(P, sampled, filters, al, st);
  if (tdt == SV_BF16 && ddt == SV_F32)
    return launch_all<uint16_t, float>(P, sampled, filters, al, st);
  return launch_all<uint16_t, uint16_t>(P, sampled, filters, al, st);
}

constexpr int MAX_BATCH = 64 * 16;   // requests a wave finds its request among

static bool grid_ok(int batch, int max_k, int nc) {
  // strips of one chunk are the worst case
  const long long g = (long long)batch * (max_k + 1) * nc + (long long)batch * nc;
  return batch <= MAX_BATCH && g < (1LL << 31);
}

static void carve(Params& P, void* ws, const Layout& L) {
  char* w = (char*)ws;
  P.cst = (u64*)(w + L.cst);
  P.dst = (u64*)(w + L.dst);
  P.rx = (u64*)(w + L.rx);
  P.dec = (u64*)(w + L.dec);
  P.res = (u64*)(w + L.res);
  P.thr_t = (u64*)(w + L.thr_t);
  P.thr_d = (u64*)(w + L.thr_d);
  P.pq = (u64*)(w + L.pq);
  P.ctl = (u64*)(w + L.ctl);
  P.order = (int32_t*)(w + L.order);
  P.okb = (int32_t*)(w + L.okb);
}


// ---------------------------------------------------------------------------
// the scratch array of the allocation-free entry point
// ---------------------------------------------------------------------------
// One array per GPU, zero-filled by the loader and again, over the bytes a
// call uses, by every call before its verify kernel.  In host code `scratch`
// names a host-side stand-in: the device address comes from
// hipGetSymbolAddress, once per device, and only that address is passed on.
constexpr size_t SCRATCH_BYTES = (size_t)8 << 20;
static __device__ __align__(256) unsigned char scratch[SCRATCH_BYTES];

constexpr int MAX_DEVICES = 64;
static std::mutex g_scratch_mu;
static void* g_scratch_ptr[MAX_DEVICES];

// Device address of the current device's scratch array, or nullptr.
static void* scratch_of_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEVICES) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}

static int fill_zero(void* p, size_t nbytes, hipStream_t st) {
  const size_t n16 = nbytes / 16;
  const size_t ntail = nbytes - n16 * 16;
  unsigned blocks = (unsigned)((n16 + 255) / 256);
  if (blocks > 4096) blocks = 4096;
  if (blocks == 0) blocks = 1;
  hipLaunchKernelGGL(k_fill_zero, dim3(blocks), dim3(256), 0, st, (uint4*)p, n16,
                     (unsigned char*)p + n16 * 16, ntail);
  return hipGetLastError() == hipSuccess ? SV_OK : SV_ERR_LAUNCH;
}

// The penalty inputs of the penalized entry point.
struct Penalties {
  const float* presence;
  const float* frequency;
  const int32_t* hist_offsets;
  const int32_t* hist_tokens;
  const int32_t* hist_counts;
  int64_t hist_nnz;
  void* penalized;
};

// The sampled verify with a caller's workspace, or (noalloc) with the
// current device's scratch array, cleared first over the bytes it needs.
static int sampled_call(const void* target_logits, int target_dtype, int64_t ld_target,
                        const void* draft, int draft_dtype, int64_t ld_draft,
                        const int32_t* draft_kind, const int32_t* cu_seqlens,
                        const int32_t* draft_tokens, const float* uniforms,
                        const float* temperature, const int32_t* top_k, const float* top_p,
                        int batch, int total_rows, int max_k, int vocab, int32_t* accepted,
                        int32_t* out_tokens, float* p_at_draft, float* q_at_draft,
                        int32_t* status, void* workspace, size_t workspace_bytes, bool noalloc,
                        void* stream, const Penalties* pen = nullptr) {
  if (!target_logits || !draft_kind || !cu_seqlens || !uniforms || !temperature || !accepted ||
      !out_tokens || !status)
    return SV_ERR_NULL;
  if (pen) {
    if (!pen->presence || !pen->frequency || !pen->penalized) return SV_ERR_NULL;
    if (pen->hist_nnz < 0 || pen->hist_nnz > INT32_MAX) return SV_ERR_SHAPE;
    if (pen->hist_nnz > 0 && (!pen->hist_offsets || !pen->hist_tokens || !pen->hist_counts))
      return SV_ERR_NULL;
  }
  if (!draft_tokens && total_rows > batch) return SV_ERR_NULL;
  if (target_dtype != SV_F32 && target_dtype != SV_BF16) return SV_ERR_DTYPE;
  if (draft && draft_dtype != SV_F32 && draft_dtype != SV_BF16) return SV_ERR_DTYPE;
  Layout L;
  int nc;
  if (!layout(batch, total_rows, vocab, max_k, L, nc) || ld_target < vocab ||
      (draft && ld_draft < vocab) || !grid_ok(batch, max_k, nc))
    return SV_ERR_SHAPE;
  if (noalloc) {
    if (L.total > SCRATCH_BYTES) return SV_ERR_SCRATCH;
    workspace = scratch_of_current_device();
    if (workspace == nullptr) return SV_ERR_LAUNCH;
    workspace_bytes = SCRATCH_BYTES;
    const int rc = fill_zero(workspace, L.total, (hipStream_t)stream);
    if (rc != SV_OK) return rc;
  }
  if (workspace_bytes < L.total) return SV_ERR_WORKSPACE;
  Params P = {};
  P.target = target_logits;
  P.draft = draft;
  P.kind = draft_kind;
  P.cu = cu_seqlens;
  P.drafts = draft_tokens;
  P.u = uniforms;
  P.temp = temperature;
  P.top_k = top_k;
  P.top_p = top_p;
  P.accepted = accepted;
  P.out = out_tokens;
  P.p_at = p_at_draft;
  P.q_at = q_at_draft;
  P.status = status;
  P.ld_t = ld_target;
  P.ld_d = draft ? ld_draft : 0;
  P.batch = batch;
  P.total_rows = total_rows;
  P.max_k = max_k;
  P.vocab = vocab;
  P.nc = nc;
  P.greedy_entry = 0;
  if (pen) {
    P.pen = pen->penalized;
    P.pres = pen->presence;
    P.freq = pen->frequency;
    P.hist_off = pen->hist_nnz > 0 ? pen->hist_offsets : nullptr;
    P.hist_tok = pen->hist_tokens;
    P.hist_cnt = pen->hist_counts;
    P.hist_nnz = pen->hist_nnz;
  }
  carve(P, workspace, L);
  const bool filters = top_k != nullptr || top_p != nullptr;
  if (!filters) {
    P.thr_t = nullptr;
    P.thr_d = nullptr;
  }
  const int ddt = draft ? draft_dtype : target_dtype;
  return dispatch(P, target_dtype, ddt, true, filters, (hipStream_t)stream);
}

}  // namespace sv

using namespace sv;

extern "C" {

int spec_verify_abi_version(void) { return SPECVERIFY_ABI_VERSION; }

const char* spec_verify_status_string(int code) {
  switch (code) {
    case SV_OK: return "ok";
    case SV_ERR_NULL: return "a required pointer is NULL";
    case SV_ERR_SHAPE: return "invalid sizes (batch, total_rows, max_k, vocab or ld)";
    case SV_ERR_DTYPE: return "unknown dtype code";
    case SV_ERR_WORKSPACE: return "workspace smaller than spec_verify_workspace_bytes()";
    case SV_ERR_LAUNCH: return "kernel launch failed";
    case SV_ERR_SCRATCH: return "the call needs more than the static scratch array holds";
    case 100 + SV_ROW_OK: return "row ok";
    case 100 + SV_ROW_NONFINITE: return "row: NaN/inf logit or invalid probability";
    case 100 + SV_ROW_EMPTY: return "row: no finite logit";
    case 100 + SV_ROW_BAD_K: return "row: offsets out of range or k > max_k";
    case 100 + SV_ROW_BAD_TOKEN: return "row: draft id outside [0, vocab)";
    case 100 + SV_ROW_BAD_PARAM: return "row: bad draft kind or temperature";
    case 100 + SV_ROW_INTERNAL: return "row: internal wait ran out (re-initialise the workspace)";
    default: return "unknown code";
  }
}

size_t spec_verify_workspace_bytes(int batch, int total_rows, int vocab, int max_k) {
  Layout L;
  int nc;
  if (!layout(batch, total_rows, vocab, max_k, L, nc)) return 0;
  return L.total;
}

int spec_verify_workspace_init(void* workspace, size_t workspace_bytes, void* stream) {
  if (!workspace) return SV_ERR_NULL;
  if (workspace_bytes == 0) return SV_OK;
  return fill_zero(workspace, workspace_bytes, (hipStream_t)stream);
}

int spec_verify_greedy(const void* target_logits, int target_dtype, int64_t ld_target,
                       const int32_t* cu_seqlens, const int32_t* draft_tokens, int batch,
                       int total_rows, int max_k, int vocab, int32_t* accepted,
                       int32_t* out_tokens, int32_t* status, void* workspace,
                       size_t workspace_bytes, void* stream) {
  if (!target_logits || !cu_seqlens || !accepted || !out_tokens || !status || !workspace)
    return SV_ERR_NULL;
  if (!draft_tokens && total_rows > batch) return SV_ERR_NULL;
  if (target_dtype != SV_F32 && target_dtype != SV_BF16) return SV_ERR_DTYPE;
  Layout L;
  int nc;
  if (!layout(batch, total_rows, vocab, max_k, L, nc) || ld_target < vocab ||
      !grid_ok(batch, max_k, nc))
    return SV_ERR_SHAPE;
  if (workspace_bytes < L.total) return SV_ERR_WORKSPACE;
  Params P = {};
  P.target = target_logits;
  P.cu = cu_seqlens;
  P.drafts = draft_tokens;
  P.accepted = accepted;
  P.out = out_tokens;
  P.status = status;
  P.ld_t = ld_target;
  P.ld_d = 0;
  P.batch = batch;
  P.total_rows = total_rows;
  P.max_k = max_k;
  P.vocab = vocab;
  P.nc = nc;
  P.greedy_entry = 1;
  carve(P, workspace, L);
  P.thr_t = nullptr;
  P.thr_d = nullptr;
  return dispatch(P, target_dtype, SV_BF16, false, false, (hipStream_t)stream);
}

int spec_verify_sampled(const void* target_logits, int target_dtype, int64_t ld_target,
                        const void* draft, int draft_dtype, int64_t ld_draft,
                        const int32_t* draft_kind, const int32_t* cu_seqlens,
                        const int32_t* draft_tokens, const float* uniforms,
                        const float* temperature, const int32_t* top_k, const float* top_p,
                        int batch, int total_rows, int max_k, int vocab, int32_t* accepted,
                        int32_t* out_tokens, float* p_at_draft, float* q_at_draft,
                        int32_t* status, void* workspace, size_t workspace_bytes,
                        void* stream) {
  if (!workspace) return SV_ERR_NULL;
  return sampled_call(target_logits, target_dtype, ld_target, draft, draft_dtype, ld_draft,
                      draft_kind, cu_seqlens, draft_tokens, uniforms, temperature, top_k, top_p,
                      batch, total_rows, max_k, vocab, accepted, out_tokens, p_at_draft,
                      q_at_draft, status, workspace, workspace_bytes, false, stream);
}

int spec_verify_sampled_penalized(const void* target_logits, int target_dtype, int64_t ld_target,
                                  const void* draft, int draft_dtype, int64_t ld_draft,
                                  const int32_t* draft_kind, const int32_t* cu_seqlens,
                                  const int32_t* draft_tokens, const float* uniforms,
                                  const float* temperature, const int32_t* top_k,
                                  const float* top_p, const float* presence,
                                  const float* frequency, const int32_t* hist_offsets,
                                  const int32_t* hist_tokens, const int32_t* hist_counts,
                                  int64_t hist_nnz, void* penalized_target, int batch,
                                  int total_rows, int max_k, int vocab, int32_t* accepted,
                                  int32_t* out_tokens, float* p_at_draft, float* q_at_draft,
                                  int32_t* status, void* workspace, size_t workspace_bytes,
                                  void* stream) {
  if (!workspace) return SV_ERR_NULL;
  const Penalties pen = {presence, frequency, hist_offsets, hist_tokens, hist_counts, hist_nnz,
                         penalized_target};
  return sampled_call(target_logits, target_dtype, ld_target, draft, draft_dtype, ld_draft,
                      draft_kind, cu_seqlens, draft_tokens, uniforms, temperature, top_k, top_p,
                      batch, total_rows, max_k, vocab, accepted, out_tokens, p_at_draft,
                      q_at_draft, status, workspace, workspace_bytes, false, stream, &pen);
}

int spec_verify_sampled_noalloc(const void* target_logits, int target_dtype, int64_t ld_target,
                                const void* draft, int draft_dtype, int64_t ld_draft,
                                const int32_t* draft_kind, const int32_t* cu_seqlens,
                                const int32_t* draft_tokens, const float* uniforms,
                                const float* temperature, const int32_t* top_k,
                                const float* top_p, int batch, int total_rows, int max_k,
                                int vocab, int32_t* accepted, int32_t* out_tokens,
                                float* p_at_draft, float* q_at_draft, int32_t* status,
                                void* stream) {
  return sampled_call(target_logits, target_dtype, ld_target, draft, draft_dtype, ld_draft,
                      draft_kind, cu_seqlens, draft_tokens, uniforms, temperature, top_k, top_p,
                      batch, total_rows, max_k, vocab, accepted, out_tokens, p_at_draft,
                      q_at_draft, status, nullptr, 0, true, stream);
}

}  // extern "C"
