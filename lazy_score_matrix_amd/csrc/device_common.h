// Device helpers shared by the tile engines: exponentials, the score
// epilogue, and order-preserving top-k keys.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pw_internal.h"

namespace pw {

constexpr float kLog2e_f = 1.4426950408889634f;
constexpr double kLog2e = 1.4426950408889634074;
constexpr float kLn2_f = 0.69314718055994531f;
constexpr double kLn2 = 0.69314718055994530942;

// exp in the working precision. float: the hardware base-2 exponential
// (v_exp_f32) of x*log2(e). double: the device library's exp.
__device__ __forceinline__ float dexp(float x) { return __builtin_amdgcn_exp2f(x * kLog2e_f); }
__device__ __forceinline__ double dexp(double x) { return exp(x); }
__device__ __forceinline__ float dlog(float x) { return __builtin_amdgcn_logf(x) * kLn2_f; }
__device__ __forceinline__ double dlog(double x) { return log(x); }

template <class T>
__device__ __forceinline__ T neg_inf() { return -__builtin_huge_valf(); }
template <>
__device__ __forceinline__ double neg_inf<double>() { return -__builtin_huge_val(); }

template <class T>
__device__ __forceinline__ T ldg(const void *p, int64_t i) { return static_cast<const T *>(p)[i]; }

// Per-row part of the epilogue, loaded once per row.
template <class T>
struct RowEpi {
  T r[kMaxStages];
  T p[kMaxStages];
};

// zb: byte offset of the batch element's epilogue vectors.
template <class T>
__device__ __forceinline__ void load_row_epi(const Epi &e, int64_t i, bool valid, RowEpi<T> &re, int64_t zb) {
#pragma unroll
  for (int s = 0; s < kMaxStages; ++s) {
    T r = (T)1, p = (T)0;
    if (s < e.n_stages && e.st[s].kind == ST_AFFINE) {
      if (e.st[s].row_vec) {
        if (valid) {
          r = ldg<T>(static_cast<const char *>(e.st[s].r_vec) + zb, i);
          p = ldg<T>(static_cast<const char *>(e.st[s].p_vec) + zb, i);
        }
      } else {
        r = (T)e.st[s].r_scalar;
        p = (T)e.st[s].p_scalar;
      }
    }
    re.r[s] = r;
    re.p[s] = p;
  }
}

// Apply the stages to score s of column slot jj; colq/colo hold the staged
// column vectors as [stage][tile width].
template <class T, int BN>
__device__ __forceinline__ T apply_epi(const Epi &e, const RowEpi<T> &re, T s, const T (*colq)[BN],
                                       const T (*colo)[BN], int jj) {
#pragma unroll
  for (int st = 0; st < kMaxStages; ++st) {
    if (st < e.n_stages) {
      if (e.st[st].kind == ST_EXP) {
        s = dexp(s);
      } else if (e.st[st].col_vec) {
        s = fma(s, re.r[st] * colq[st][jj], re.p[st] + colo[st][jj]);
      } else {
        s = fma(s, re.r[st], re.p[st]);
      }
    }
  }
  return s;
}

// ---------------------------------------------------------------------------
// Top-k keys: total order (value, index), smaller first. For `largest` the
// value is negated so the same "smaller first" order applies; -0 and +0 are
// the same value. NaN is not supported.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t f32_ord(float v) {
  uint32_t b = __float_as_uint(v == 0.0f ? 0.0f : v);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
__device__ __forceinline__ float f32_from_ord(uint32_t o) {
  uint32_t b = (o & 0x80000000u) ? (o & 0x7fffffffu) : ~o;
  return __uint_as_float(b);
}
__device__ __forceinline__ uint64_t f64_ord(double v) {
  uint64_t b = (uint64_t)__double_as_longlong(v == 0.0 ? 0.0 : v);
  return (b & 0x8000000000000000ull) ? ~b : (b | 0x8000000000000000ull);
}
__device__ __forceinline__ double f64_from_ord(uint64_t o) {
  uint64_t b = (o & 0x8000000000000000ull) ? (o & 0x7fffffffffffffffull) : ~o;
  return __longlong_as_double((long long)b);
}

template <class T>
struct Key;

template <>
struct Key<float> {
  uint64_t k;
  __device__ __forceinline__ static Key make(float v, uint32_t j, int largest) {
    return Key{((uint64_t)f32_ord(largest ? -v : v) << 32) | j};
  }
  __device__ __forceinline__ static Key sentinel() { return Key{~0ull}; }
  __device__ __forceinline__ bool operator<(const Key &o) const { return k < o.k; }
  __device__ __forceinline__ float value(int largest) const {
    float v = f32_from_ord((uint32_t)(k >> 32));
    return largest ? -v : v;
  }
  __device__ __forceinline__ uint32_t index() const { return (uint32_t)k; }
  // Output index: -1 for an empty slot (fewer kept pairs than k).
  __device__ __forceinline__ int64_t out_index() const { return (uint32_t)k == ~0u ? -1 : (int64_t)(uint32_t)k; }
  __device__ __forceinline__ void store(void *base, int64_t e) const { static_cast<uint64_t *>(base)[e] = k; }
  __device__ __forceinline__ static Key load(const void *base, int64_t e) {
    return Key{static_cast<const uint64_t *>(base)[e]};
  }
};

template <>
struct Key<double> {
  uint64_t v;
  uint32_t j;
  __device__ __forceinline__ static Key make(double x, uint32_t j, int largest) {
    return Key{f64_ord(largest ? -x : x), j};
  }
  __device__ __forceinline__ static Key sentinel() { return Key{~0ull, ~0u}; }
  __device__ __forceinline__ bool operator<(const Key &o) const {
    return v < o.v || (v == o.v && j < o.j);
  }
  __device__ __forceinline__ double value(int largest) const {
    double x = f64_from_ord(v);
    return largest ? -x : x;
  }
  __device__ __forceinline__ uint32_t index() const { return j; }
  __device__ __forceinline__ int64_t out_index() const { return j == ~0u ? -1 : (int64_t)j; }
  __device__ __forceinline__ void store(void *base, int64_t e) const {
    uint64_t *b = static_cast<uint64_t *>(base);
    b[2 * e] = v;
    b[2 * e + 1] = j;
  }
  __device__ __forceinline__ static Key load(const void *base, int64_t e) {
    const uint64_t *b = static_cast<const uint64_t *>(base);
    return Key{b[2 * e], (uint32_t)b[2 * e + 1]};
  }
};

// Insert `c` into the ascending list l[0..L); the largest key falls off.
template <class T, int L>
__device__ __forceinline__ void key_insert(Key<T> (&l)[L], Key<T> c) {
  if (c < l[L - 1]) {
#pragma unroll
    for (int p = 0; p < L; ++p) {
      bool lt = c < l[p];
      Key<T> lo = lt ? c : l[p];
      Key<T> hi = lt ? l[p] : c;
      l[p] = lo;
      c = hi;
    }
  }
}

// Insert `c` into the ascending list l[0..L) when every key already in it
// has a smaller index (keys reach the list in increasing column order), so
// that c belongs right after the last key of smaller or equal value: only
// the values are compared, and each slot takes its left neighbour, c, or
// itself. The caller has checked that c enters (its value is below the last
// slot's). For float keys the value is the high word; double keys take the
// full compare-swap pass.
template <int L>
__device__ __forceinline__ void key_insert_after(Key<float> (&l)[L], Key<float> c) {
  const uint32_t cv = (uint32_t)(c.k >> 32);
  bool lt[L];
#pragma unroll
  for (int p = 0; p < L; ++p) lt[p] = cv < (uint32_t)(l[p].k >> 32);
#pragma unroll
  for (int p = L - 1; p > 0; --p) l[p].k = lt[p - 1] ? l[p - 1].k : (lt[p] ? c.k : l[p].k);
  l[0].k = lt[0] ? c.k : l[0].k;
}
template <int L>
__device__ __forceinline__ void key_insert_after(Key<double> (&l)[L], Key<double> c) {
  if (c < l[L - 1]) {
#pragma unroll
    for (int p = 0; p < L; ++p) {
      bool lt = c < l[p];
      Key<double> lo = lt ? c : l[p];
      Key<double> hi = lt ? l[p] : c;
      l[p] = lo;
      c = hi;
    }
  }
}

// The arrays of batch element blockIdx.z, each offset by its batch stride
// (element 0, and every unbatched launch, see them as given). Kernels read
// their arrays through these; the epilogue's stage vectors are offset where
// they are read (epi_vec).
// (The host gives an absent array, a null pointer, stride 0.)
__device__ __forceinline__ const void *batch_ptr(const void *p, int64_t stride, int64_t z) {
  return static_cast<const char *>(p) + stride * z;
}
__device__ __forceinline__ void *batch_ptr(void *p, int64_t stride, int64_t z) {
  return static_cast<char *>(p) + stride * z;
}
struct BatchPtrs {
  const void *X, *Y, *V, *ny;
  void *out, *lse_out, *partial;
  int64_t *idx;
};
__device__ __forceinline__ BatchPtrs batch_ptrs(const TileArgs &a) {
  const int64_t z = blockIdx.z;
  BatchPtrs b;
  b.X = batch_ptr(a.X, a.bat.x, z);
  b.Y = batch_ptr(a.Y, a.bat.y, z);
  b.V = batch_ptr(a.V, a.bat.v, z);
  b.ny = batch_ptr(a.ny, a.bat.ny, z);
  b.out = batch_ptr(a.out, a.bat.out, z);
  b.lse_out = batch_ptr(a.lse_out, a.bat.lse, z);
  b.partial = batch_ptr(a.partial, a.bat.part, z);
  b.idx = static_cast<int64_t *>(batch_ptr(static_cast<void *>(a.idx), a.bat.idx, z));
  return b;
}
// Byte offset of this batch element's epilogue vectors, and one of them.
__device__ __forceinline__ int64_t epi_shift(const TileArgs &a) { return a.bat.epi * (int64_t)blockIdx.z; }
__device__ __forceinline__ const void *epi_vec(const TileArgs &a, const void *v) {
  return static_cast<const char *>(v) + epi_shift(a);
}

// A value known to be equal on every lane, moved to scalar registers.
__device__ __forceinline__ int64_t wave_uniform(int64_t v) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)(uint64_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)v >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

// A compile-time flag passed as a value (to generic lambdas).
template <bool B>
struct Bool {
  static constexpr bool value = B;
};

// ------------------------------------------------------------------ masks
// Tile classes under the pair masks, for the rows r0..r1 of a row block and
// the keys j0..j1 of a tile (both inclusive, non-empty).
enum TileClass : int { TILE_SKIP = 0, TILE_CHECK = 1, TILE_FULL = 2 };

__device__ __forceinline__ int tile_class(const MaskArgs &m, int64_t r0, int64_t r1, int64_t j0, int64_t j1,
                                          int rb, int64_t tile) {
  int c = TILE_FULL;
  if (m.band) {
    // j - i spans [j0 - r1, j1 - r0] over the tile.
    if (j1 - r0 < m.lo || j0 - r1 > m.hi) return TILE_SKIP;
    if (j0 - r1 < m.lo || j1 - r0 > m.hi) c = TILE_CHECK;
  }
  if (m.grow) {
    const int64_t a0 = m.grow_rng[2 * rb], a1 = m.grow_rng[2 * rb + 1];
    const int64_t b0 = m.gcol_rng[2 * tile], b1 = m.gcol_rng[2 * tile + 1];
    if (b1 < a0 || b0 > a1) return TILE_SKIP;
    if (!(a0 == a1 && b0 == b1 && a0 == b0)) c = TILE_CHECK;
  }
  if (m.col) c = TILE_CHECK;
  return c;
}

// The key range [first, last) row block rb (rows r0..r1) visits inside the
// column split [jb, je): the band's reach, cut to the block's span of kept
// tiles when one was computed, with `first` on a tile boundary.
__device__ __forceinline__ void band_range(const MaskArgs &m, int rb, int64_t r0, int64_t r1, int64_t jb, int64_t je,
                                           int bn, int64_t *first, int64_t *last) {
  int64_t f = jb, l = je;
  if (m.band) {
    const int64_t lo = r0 + m.lo, hi = r1 + m.hi + 1;
    if (lo > jb) f = jb + (lo - jb) / bn * bn;
    l = min(l, hi);
  }
  if (m.span) {
    const int64_t s0 = m.span[2 * rb], s1 = m.span[2 * rb + 1];
    if (s0 > f) f = jb + (s0 - jb) / bn * bn;
    l = min(l, s1);
  }
  *first = f;
  *last = l;
}

// Whether pair (i, j) survives the band and the group mask (the column mask
// is staged per key by the engines).
__device__ __forceinline__ bool pair_kept(const MaskArgs &m, int64_t i, int64_t j, int64_t gi, int64_t gj) {
  const int64_t d = j - i;
  return (!m.band || (d >= m.lo && d <= m.hi)) && (!m.grow || gi == gj);
}

// Top-k filter threshold: the signed value (negated for `largest`) of the
// list's last key, +inf while that slot is empty. Within one lane (or one
// thread) keys arrive in increasing column order, so a candidate whose value
// equals the threshold loses the index tie-break and is rightly skipped by a
// strict <.
__device__ __forceinline__ float key_threshold(const Key<float> &last) {
  const uint32_t hi = (uint32_t)(last.k >> 32);
  return hi == 0xffffffffu ? __builtin_huge_valf() : f32_from_ord(hi);
}
__device__ __forceinline__ double key_threshold(const Key<double> &last) {
  return last.v == ~0ull ? __builtin_huge_val() : f64_from_ord(last.v);
}

}  // namespace pw
