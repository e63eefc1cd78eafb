// nha_common.h -- device helpers shared by the NHA kernels (gfx950 only).
//
// Matrix-core conventions used throughout (one 64-lane wavefront, lane l,
// g = l / 16, c = l % 16):
//   16x16 accumulator D (4 floats per lane):  lane l holds D[4g + r][c], r=0..3
//   K=32 step (v_mfma_f32_16x16x32_bf16):      A frag = A[c][8g .. 8g+7]
//                                             B frag = B[8g .. 8g+7][c]
//   K=16 step (v_mfma_f32_16x16x16_bf16):      A frag = A[c][4g .. 4g+3]
//                                             B frag = B[4g .. 4g+3][c]
// For float operands the same per-lane fragments (8 or 4 consecutive k) are fed
// to v_mfma_f32_16x16x4_f32 one k at a time: instruction s uses element s of
// every lane, i.e. the k-subset {s, 8+s, 16+s, 24+s} (resp. {s, 4+s, ...}).
// Summation over k is order-free, so both element types share every fragment
// layout and every kernel is written once for T in {float, __bf16}.
//
// Because the K index of a step may be any permutation applied to both
// operands, an accumulator tile in D layout (lane l holds rows 4g..4g+3 of
// column c) can feed the next product directly as a B fragment:
//   K=16: the 4 values themselves;   K=32: rows {4g+r} of block 2s and
//   {4g+r} of block 2s+1, with the A fragment read in the same order
//   (A[c][32s + 4g + r] and A[c][32s + 16 + 4g + r]).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

typedef __bf16 bf16;
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx8 __attribute__((ext_vector_type(8)));
typedef bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef bf16 bf16x8 __attribute__((ext_vector_type(8)));
// fp16: 10 mantissa bits for [0, 1]-bounded or moderate fp32 tiles handed
// between kernels (the bf16 MFMA operands they end up in keep 7)
typedef _Float16 f16;
typedef f16 f16x4 __attribute__((ext_vector_type(4)));

#define NHA_LOG2E 1.4426950408889634f
#define NHA_LN2 0.6931471805599453f
// Floor of log2(alpha): gates below 2^-80 decay like 2^-80 (their slot is
// overwritten to within 1e-24 relative either way); keeps every exponent
// difference finite.
#define NHA_LOG2A_MIN (-80.0f)

template <typename T> struct Vec;
template <> struct Vec<bf16> { typedef bf16x8 v8; typedef bf16x4 v4; };
template <> struct Vec<float> { typedef floatx8 v8; typedef floatx4 v4; };

__device__ __forceinline__ floatx4 zero4() { return floatx4{0.f, 0.f, 0.f, 0.f}; }

// ---------------------------------------------------------------- MFMA steps
__device__ __forceinline__ floatx4 mma32(floatx4 acc, bf16x8 a, bf16x8 b) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc, 0, 0, 0);
}
__device__ __forceinline__ floatx4 mma32(floatx4 acc, floatx8 a, floatx8 b) {
#pragma unroll
  for (int s = 0; s < 8; ++s) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[s], b[s], acc, 0, 0, 0);
  return acc;
}
__device__ __forceinline__ floatx4 mma16(floatx4 acc, bf16x4 a, bf16x4 b) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, acc, 0, 0, 0);
}
__device__ __forceinline__ floatx4 mma16(floatx4 acc, floatx4 a, floatx4 b) {
#pragma unroll
  for (int s = 0; s < 4; ++s) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[s], b[s], acc, 0, 0, 0);
  return acc;
}

// ---------------------------------------------------------------- conversions
template <typename T> __device__ __forceinline__ T to_t(float x);
template <> __device__ __forceinline__ float to_t<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16 to_t<bf16>(float x) { return (bf16)x; }

template <typename T> __device__ __forceinline__ float to_f(T x) { return (float)x; }

// Pack 8 floats into a fragment of T.
template <typename T>
__device__ __forceinline__ typename Vec<T>::v8 pack8(const float* f) {
  typename Vec<T>::v8 r;
#pragma unroll
  for (int i = 0; i < 8; ++i) r[i] = to_t<T>(f[i]);
  return r;
}
template <typename T>
__device__ __forceinline__ typename Vec<T>::v8 pack8(floatx4 a, floatx4 b) {
  typename Vec<T>::v8 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    r[i] = to_t<T>(a[i]);
    r[4 + i] = to_t<T>(b[i]);
  }
  return r;
}
template <typename T>
__device__ __forceinline__ typename Vec<T>::v4 pack4(floatx4 a) {
  typename Vec<T>::v4 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) r[i] = to_t<T>(a[i]);
  return r;
}

// ---------------------------------------------------------------- loads / stores
template <typename T>
__device__ __forceinline__ typename Vec<T>::v4 ld4(const T* p) {
  return *reinterpret_cast<const typename Vec<T>::v4*>(p);
}
// 8 consecutive elements (16-byte aligned; float is read as two halves so
// that 16-byte alignment suffices for it as well).
template <typename T>
__device__ __forceinline__ typename Vec<T>::v8 ld8(const T* p) {
  if constexpr (sizeof(T) == 2) {
    return *reinterpret_cast<const typename Vec<T>::v8*>(p);
  } else {
    typename Vec<T>::v4 a = ld4<T>(p), b = ld4<T>(p + 4);
    typename Vec<T>::v8 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      r[i] = a[i];
      r[4 + i] = b[i];
    }
    return r;
  }
}
// Two groups of 4 consecutive elements -> one K=32 fragment (permuted order).
template <typename T>
__device__ __forceinline__ typename Vec<T>::v8 ld4x2(const T* p0, const T* p1) {
  typename Vec<T>::v4 a = ld4(p0), b = ld4(p1);
  typename Vec<T>::v8 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    r[i] = a[i];
    r[4 + i] = b[i];
  }
  return r;
}
template <typename T>
__device__ __forceinline__ void st8(T* p, typename Vec<T>::v8 v) {
  *reinterpret_cast<typename Vec<T>::v8*>(p) = v;
}
template <typename T>
__device__ __forceinline__ void st4(T* p, typename Vec<T>::v4 v) {
  *reinterpret_cast<typename Vec<T>::v4*>(p) = v;
}
template <typename T>
__device__ __forceinline__ typename Vec<T>::v8 zero8() {
  typename Vec<T>::v8 r;
#pragma unroll
  for (int i = 0; i < 8; ++i) r[i] = to_t<T>(0.f);
  return r;
}
// 8 elements at p when ok, else zeros.  The load itself is unconditional, so
// p must be readable either way (callers clamp the row): a load under a branch
// makes the compiler wait for it before the branch joins, which serialises
// every load issued before it.
template <typename T>
__device__ __forceinline__ typename Vec<T>::v8 ld8_sel(const T* p, bool ok) {
  const typename Vec<T>::v8 v = ld8<T>(p);
  return ok ? v : zero8<T>();
}

// Buffer-resource loads: a resource covers [p, p + bytes) and a load whose
// offset falls outside returns zeros without touching memory, so ragged tile
// edges need neither branches nor masks (the offset is unsigned: a row before
// the covered range wraps to a huge offset and reads as zeros too).  The
// resource lives in SGPRs: p and bytes must be uniform over the wave.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void* p, uint32_t bytes) {
  const uintptr_t a = (uintptr_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a),
                 hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  return __builtin_amdgcn_make_buffer_rsrc((void*)(((uintptr_t)hi << 32) | lo), (short)0,
                                           (int)__builtin_amdgcn_readfirstlane(bytes), 0x00020000);
}
// 16 bytes at byte offset off
__device__ __forceinline__ bf16x8 buf_ld16(__amdgpu_buffer_rsrc_t r, uint32_t off, bf16x8*) {
  return __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
__device__ __forceinline__ floatx8 buf_ld16(__amdgpu_buffer_rsrc_t r, uint32_t off, floatx8*) {
  const floatx4 a = __builtin_bit_cast(floatx4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
  const floatx4 b = __builtin_bit_cast(floatx4, __builtin_amdgcn_raw_buffer_load_b128(r, off + 16, 0, 0));
  floatx8 v;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[i] = a[i];
    v[4 + i] = b[i];
  }
  return v;
}
// 8 elements of T at element offset off (zeros outside the resource)
template <typename T>
__device__ __forceinline__ typename Vec<T>::v8 buf_ld8(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return buf_ld16(r, off * (uint32_t)sizeof(T), (typename Vec<T>::v8*)nullptr);
}
// Resource over rows [lo, hi) of a row-major tile with leading dimension ld
// (elements), clipped to [0, rows): element (rr, j) sits at element offset
// (rr - max(lo, 0)) * ld + j.
template <typename T>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rows_rsrc(const T* base, size_t ld, int lo, int hi, int rows,
                                                           int width, int& first) {
  first = lo > 0 ? lo : 0;
  const int last = hi < rows ? hi : rows;
  const uint32_t bytes = last > first ? (uint32_t)(((size_t)(last - first - 1) * ld + width) * sizeof(T)) : 0u;
  return buf_rsrc(base + (size_t)first * ld, bytes);
}

// 8 consecutive elements converted to float.
template <typename T>
__device__ __forceinline__ void ld8f(const T* p, float* f) {
  typename Vec<T>::v8 v = ld8<T>(p);
#pragma unroll
  for (int i = 0; i < 8; ++i) f[i] = to_f<T>(v[i]);
}

// ---------------------------------------------------------------- cross-lane
__device__ __forceinline__ float shfl_xor(float x, int m) { return __shfl_xor(x, m, 64); }
// Reduce over the 4 lane groups g (lanes c, c+16, c+32, c+48).
__device__ __forceinline__ float max_over_g(float x) {
  x = fmaxf(x, shfl_xor(x, 16));
  return fmaxf(x, shfl_xor(x, 32));
}
__device__ __forceinline__ float sum_over_g(float x) {
  x += shfl_xor(x, 16);
  return x + shfl_xor(x, 32);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Combine a value with the one held by lane l ^ 32 (v_permlane32_swap: the
// pair returned holds both halves' values in either lane, in some order).
__device__ __forceinline__ float max_halves(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_halves(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Workgroups are dispatched round-robin over the 8 XCDs of an MI355X (linear
// id n goes to XCD n % 8), and each XCD has its own L2.  xcd_remap turns the
// linear id into a logical index such that every XCD receives one contiguous
// range of logical indices: neighbouring tiles (which share K/V rows) then run
// on the same XCD and hit its L2.  Bijective on [0, N).
__device__ __forceinline__ int xcd_remap(int lin, int N) {
  int q = N >> 3, r = N & 7, x = lin & 7, k = lin >> 3;
  return x * q + (x < r ? x : r) + k;
}

// Padded row pitch (elements) for LDS tiles of T with `cols` columns: keeps
// 16-byte alignment and shifts consecutive rows across banks.
__host__ __device__ constexpr int pitch_of(int cols) { return cols + 8; }

// ---------------------------------------------------------------- tile staging
// A ROWS-row tile of a row-major [rows][D] operand (row stride `ld` elements);
// rows outside [lo, hi) read as zero.  NT threads; each thread owns 8-element
// chunks.  load() issues the global loads into registers (so they can overlap
// other work), store() writes them to LDS.
template <typename T, int D, int NT, int ROWS = 64>
struct RowTile {
  static constexpr int CH = ROWS * D / 8;         // 8-element chunks per tile
  static constexpr int PER = (CH + NT - 1) / NT;  // chunks per thread
  typename Vec<T>::v8 r[PER];
  // rows rr in [lo, hi) (and < ROWS) are read, the others are zero
  __device__ __forceinline__ void load(const T* __restrict__ base, size_t ld, int lo, int hi, int tid) {
    int first;
    const __amdgpu_buffer_rsrc_t rs = rows_rsrc<T>(base, ld, lo, hi, ROWS, D, first);
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int e = (tid + k * NT) * 8, rr = e / D, j = e % D;
      r[k] = buf_ld8<T>(rs, (uint32_t)((rr - first) * (int)ld + j));
    }
  }
  // LDS layout [ROWS][P] (P = row pitch in elements)
  template <int P>
  __device__ __forceinline__ void store(T* lds, int tid) const {
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      int e = (tid + k * NT) * 8;
      if (e < ROWS * D) st8<T>(lds + (e / D) * P + (e % D), r[k]);
    }
  }
};

// A [ROWS][D] tile kept in HBM in column blocks of 16, [D / 16][ROWS][16]
// (what a scan wave owning 16 columns writes contiguously), loaded with
// contiguous 16-byte pieces and stored to LDS in row layout [ROWS][P].
template <typename T, int D, int NT, int ROWS>
struct BlockedTile {
  static constexpr int CH = ROWS * D / 8;
  static constexpr int PER = (CH + NT - 1) / NT;
  typename Vec<T>::v8 r[PER];
  __device__ __forceinline__ void load(const T* __restrict__ src, int tid) {
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int q = tid + k * NT;
      r[k] = ld8<T>(src + 8 * (q < CH ? q : CH - 1));
    }
  }
  template <int P>
  __device__ __forceinline__ void store(T* lds, int tid) const {
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int q = tid + k * NT, e = 8 * q, jb = e / (ROWS * 16), rem = e % (ROWS * 16);
      if (q < CH) st8<T>(lds + (rem / 16) * P + 16 * jb + (rem % 16), r[k]);
    }
  }
};

// Position of row k inside a transposed row when SWZ is set: bits 2 and 3 of
// k trade places, so that within every 16-row group the rows {4h + r} and
// {8 + 4h + r} (h = 0, 1; r = 0..3) -- the K=16 step of a 32x32 product fed
// from an accumulator in D layout -- sit next to each other at 8h .. 8h+7.
__host__ __device__ constexpr int kswz(int k) { return (k & ~12) | ((k & 4) << 1) | ((k & 8) >> 1); }

// The same tile stored transposed ([D][P], row index contiguous), for operands
// whose K dimension is the tile's row index.  Thread = (row pair p, column-chunk
// group): it loads rows 2p and 2p+1 of one 8-column chunk and writes 8 packed
// pairs, so a wavefront writes consecutive pairs of one LDS row per store
// (conflict-free) instead of scattering 2-byte values.  With SWZ the pair of
// rows 2p, 2p+1 lands at kswz(2p) (the swap keeps pairs together).
template <typename T, int D, int NT, int ROWS = 64, bool SWZ = false>
struct PairTileT {
  static constexpr int NP = ROWS / 2;                // row pairs
  static constexpr int NG = NT / NP;                 // chunk groups
  static constexpr int NCH = D / 8;                  // 8-column chunks
  static constexpr int PER = (NCH + NG - 1) / NG;    // chunks per thread
  typename Vec<T>::v8 a[PER], b[PER];
  __device__ __forceinline__ void load(const T* __restrict__ base, size_t ld, int lo, int hi, int tid) {
    const int p = tid % NP, cg = tid / NP;
    int first;
    const __amdgpu_buffer_rsrc_t rs = rows_rsrc<T>(base, ld, lo, hi, ROWS, D, first);
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int c = cg + k * NG, cl = c < NCH ? c : NCH - 1;
      a[k] = buf_ld8<T>(rs, (uint32_t)((2 * p - first) * (int)ld + 8 * cl));
      b[k] = buf_ld8<T>(rs, (uint32_t)((2 * p + 1 - first) * (int)ld + 8 * cl));
    }
  }
  template <int P>
  __device__ __forceinline__ void store(T* lds, int tid) const {
    int p = tid % NP, cg = tid / NP;
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      int c = cg + k * NG;
      if (c < NCH && cg < NG) {
        const int col = SWZ ? kswz(2 * p) : 2 * p;
        const typename Vec<T>::v8 ak = a[k], bk = b[k];
        if constexpr (sizeof(T) == 2) {
          // bf16: word x/2 of each row holds columns x (low half) and x+1
          typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
          u32x4 wa = __builtin_bit_cast(u32x4, ak), wb = __builtin_bit_cast(u32x4, bk);
#pragma unroll
          for (int x = 0; x < 8; ++x) {
            uint32_t v = __builtin_amdgcn_perm(wb[x >> 1], wa[x >> 1], (x & 1) ? 0x07060302u : 0x05040100u);
            *reinterpret_cast<uint32_t*>(lds + (8 * c + x) * P + col) = v;
          }
        } else {
#pragma unroll
          for (int x = 0; x < 8; ++x) {
            typedef T pair_t __attribute__((ext_vector_type(2)));
            pair_t v;
            v[0] = ak[x];
            v[1] = bk[x];
            *reinterpret_cast<pair_t*>(lds + (8 * c + x) * P + col) = v;
          }
        }
      }
    }
  }
};

// ---------------------------------------------------------------- 32x32 tiles
// 32x32 accumulator (16 floats per lane, h = l / 32, c = l % 32):
//   lane l holds D[8 (r / 4) + 4 h + r % 4][c], r = 0..15
// K=16 step (v_mfma_f32_32x32x16_bf16): A frag = A[c][8h .. 8h+7],
//                                      B frag = B[8h .. 8h+7][c]
// Float operands use v_mfma_f32_32x32x2_f32 once per element s of the same
// fragments (k-subset {s, 8 + s}).
typedef float floatx16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ floatx16 zero16() {
  floatx16 r;
#pragma unroll
  for (int i = 0; i < 16; ++i) r[i] = 0.f;
  return r;
}
__device__ __forceinline__ floatx16 mma32x32(floatx16 acc, bf16x8 a, bf16x8 b) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc, 0, 0, 0);
}
__device__ __forceinline__ floatx16 mma32x32(floatx16 acc, floatx8 a, floatx8 b) {
#pragma unroll
  for (int s = 0; s < 8; ++s) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a[s], b[s], acc, 0, 0, 0);
  return acc;
}
// 8 consecutive accumulator entries r0 .. r0+7 packed as one fragment of T.
template <typename T>
__device__ __forceinline__ typename Vec<T>::v8 pack8_at(const floatx16& a, int r0) {
  typename Vec<T>::v8 r;
#pragma unroll
  for (int i = 0; i < 8; ++i) r[i] = to_t<T>(a[r0 + i]);
  return r;
}

// ---------------------------------------------------------------- direct-to-LDS staging (bf16)
// 64-row bf16 tiles kept unpadded in LDS ([row][D], rows of D/8 16-byte
// chunks) and filled with global_load_lds_dwordx4: every wave instruction
// writes 64 x 16 contiguous bytes (lane l at byte 16 l), i.e. 64 / (D/8)
// whole rows.  The chunk order inside a row is permuted (XOR with a function
// of the row) so that the two read patterns below meet every bank once:
//   kind 0 (row-major fragments): lane c reads one chunk of row r0 + c
//   kind 1 (transposed reads):    16 lanes read 2 neighbouring chunks of 4
//                                 consecutive rows (ds_read_b64_tr_b16)
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void glb_void_t;
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4_t;

//   kind 2 (both of the above) on gfx950's 64 banks x 4 bytes, where a
//                                 16-byte read serves 16 lanes (256 bytes) per
//                                 pass and a ds_read_b64_tr_b16 32 lanes:
//     D = 128 (a row fills the 64 banks): f(r) = 4 (r % 4) + (r / 4) % 4 is a
//       permutation of the 16 chunk positions over 16 consecutive rows (row
//       reads), and gives 4 aligned rows 4 different 4-chunk groups (the 4
//       chunks each such row gives a transposed read);
//     D = 64 (two rows per 64 banks): f(r) = 4 ((r / 2) % 2) + (r / 4) % 4 is
//       distinct over the 8 even (and the 8 odd) rows of 16, and puts rows r
//       and r + 2 of an aligned 4 (same bank half) in different 4-chunk groups;
//     D = 32 (four rows per 64 banks): f(r) = (r / 4) % 4 is distinct over the
//       4 rows of 16 that share a bank quarter; transposed reads of 4 aligned
//       rows fall in 4 different quarters whatever the permutation.
//   kind 3 (both, repeating every 8 rows, so that a transposed read can
//                                 reach the second group of 8 rows with a
//                                 constant offset): the transposed condition
//                                 above holds, row reads are 2-way:
//     D = 128: 4 (r % 4) + (r / 4) % 2;  D = 64: 4 ((r / 2) % 2) + 2 (r % 2) +
//     (r / 4) % 2;  D = 32: (r / 4) % 2.
//   (The kinds 0 and 1 satisfy the same conditions for one pattern each; kind
//   2 repeats every 16 rows.)
template <int D, int KIND>
__device__ __forceinline__ int chunk_swz(int row) {
  if constexpr (KIND == 0) return row & (D / 8 - 1);
  else if constexpr (KIND == 1) return ((0xAC60 >> (4 * (row & 3))) & 15) & (D / 8 - 1);
  else if constexpr (KIND == 2) {
    if constexpr (D >= 128) return (((row & 3) << 2) | ((row >> 2) & 3)) & (D / 8 - 1);
    else if constexpr (D == 64) return ((((row >> 1) & 1) << 2) | ((row >> 2) & 3)) & (D / 8 - 1);
    else return ((row >> 2) & 3) & (D / 8 - 1);
  } else {
    if constexpr (D >= 128) return (((row & 3) << 2) | ((row >> 2) & 1)) & (D / 8 - 1);
    else if constexpr (D == 64) return ((((row >> 1) & 1) << 2) | ((row & 1) << 1) | ((row >> 2) & 1)) & (D / 8 - 1);
    else return ((row >> 2) & 1) & (D / 8 - 1);
  }
}

// Rows [j0, j0 + 64) of a bf16 operand with row stride ld (rows past Tn - 1
// repeat row Tn - 1; callers mask those keys) into the swizzled tile `lds`.
// NT threads; each wave issues D/8 / (NT/64) instructions.
template <int D, int NT, int KIND>
__device__ __forceinline__ void dma_tile(const bf16* __restrict__ base, size_t ld, int j0, int Tn, bf16* lds,
                                         int tid) {
  constexpr int CPR = D / 8, RPI = 64 / CPR, NI = 64 / RPI, NW = NT / 64;
  const int wv = tid >> 6, l = tid & 63;
#pragma unroll
  for (int i0 = 0; i0 < NI; i0 += NW) {
    const int i = i0 + wv;
    if (NI % NW == 0 || i < NI) {
      const int r = i * RPI + l / CPR;
      const int q = (l % CPR) ^ chunk_swz<D, KIND>(r);
      const int gr = min(j0 + r, Tn - 1);
      __builtin_amdgcn_global_load_lds((glb_void_t*)(base + (size_t)gr * ld + 8 * q),
                                       (lds_void_t*)(lds + i * RPI * D), 16, 0, 0);
    }
  }
}

// A wave's 32 x D bf16 output tile in the 32x32 MFMA layout (lane (hf, c)
// holds row c, columns 32 dt + 8 i + 4 hf + r as val(dt, 4 i + r)) goes out
// through LDS: the lanes put 8-byte pieces into the wave's staging area stg
// (32 rows, pitch D + 4: the 8-byte writes of a half-wave hit distinct banks),
// then each lane writes 16 bytes of one row, so that every store instruction
// covers whole rows.  out + row_off(r) receives row r (plus add + row_off(r)
// when add_row(r)), for rows r with r < nrows.  stg is private to the wave;
// on return its reads are complete.
template <int D, typename Val, typename RowOff, typename AddRow>
__device__ __forceinline__ void store_tile_rows(Val val, bf16* stg, bf16* __restrict__ out,
                                                const bf16* __restrict__ add, RowOff row_off, AddRow add_row,
                                                int nrows) {
  constexpr int PS = D + 4, CPR = D / 8, RPI = 64 / CPR;
  const int l = threadIdx.x & 63, hf = l >> 5, c = l & 31;
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const floatx4 x{val(dt, 4 * i), val(dt, 4 * i + 1), val(dt, 4 * i + 2), val(dt, 4 * i + 3)};
      st4<bf16>(stg + c * PS + 32 * dt + 8 * i + 4 * hf, pack4<bf16>(x));
    }
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
  for (int k = 0; k < 32 / RPI; ++k) {
    const int row = RPI * k + l / CPR, q = l % CPR;
    const bf16x4 a0 = *reinterpret_cast<const bf16x4*>(stg + row * PS + 8 * q);
    const bf16x4 a1 = *reinterpret_cast<const bf16x4*>(stg + row * PS + 8 * q + 4);
    if (row < nrows) {
      const size_t ro = row_off(row) + 8 * q;
      float y[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        y[e] = (float)a0[e];
        y[4 + e] = (float)a1[e];
      }
      if (add != nullptr && add_row(row)) {
        const bf16x8 z = ld8<bf16>(add + ro);
#pragma unroll
        for (int e = 0; e < 8; ++e) y[e] += (float)z[e];
      }
      st8<bf16>(out + ro, pack8<bf16>(floatx4{y[0], y[1], y[2], y[3]}, floatx4{y[4], y[5], y[6], y[7]}));
    }
  }
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
}

// Wait for this wave's outstanding global loads (including the ones that
// write LDS directly); a barrier must follow before other waves read them.
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

__device__ __forceinline__ bf16x4 ld_tr4(const bf16* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t*)p);
}
// The same reads from a 32-bit LDS byte address.
typedef __attribute__((address_space(3))) bf16x8 lds_bf16x8_t;
__device__ __forceinline__ bf16x4 ld_tr4_at(uint32_t a) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t*)(uintptr_t)a);
}
__device__ __forceinline__ bf16x8 ld8_at(uint32_t a) { return *(lds_bf16x8_t*)(uintptr_t)a; }

// The same staging issued through inline assembly, so that the compiler does
// not order later LDS reads of *other* buffers after these loads (it cannot
// tell the buffers apart).  The caller waits with wait_vmem() and a barrier
// before anyone reads the tile.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)((const lds_void_t*)p);
}
// A wave-uniform pointer as an SGPR pair.
__device__ __forceinline__ uint64_t sgpr_ptr(const void* p) {
  const uint64_t v = (uint64_t)(uintptr_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v), hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return ((uint64_t)hi << 32) | lo;
}
// Per-lane part (bytes) of the source offset of this wave's instructions
// relative to their first row; callers compute it once and pass it in.
template <int D, int NT, int KIND>
__device__ __forceinline__ uint32_t dma_lane_off(int tid, size_t ld) {
  constexpr int CPR = D / 8, RPI = 64 / CPR;
  const int wv = tid >> 6, l = tid & 63;
  const int r = wv * RPI + l / CPR;
  const int q = (l % CPR) ^ chunk_swz<D, KIND>(r);
  return (uint32_t)((l / CPR) * ld * 2 + 16 * q);
}
template <int D, int NT, int KIND>
__device__ __forceinline__ void dma_tile_async(const bf16* __restrict__ base, size_t ld, int j0, int Tn,
                                               uint32_t lds, uint32_t loff, int tid) {
  constexpr int CPR = D / 8, RPI = 64 / CPR, NI = 64 / RPI, NW = NT / 64;
  static_assert(NI % NW == 0, "tile instructions must split evenly over the waves");
  // rows NW RPI apart share their swizzle, so one lane offset serves every
  // instruction of the wave
  static_assert((NW * RPI) % (KIND == 0 ? CPR : KIND == 1 ? 4 : 8) == 0, "swizzle period");
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6), l = tid & 63;
  if (j0 + 64 <= Tn) {
    // whole tile in range: uniform row base in SGPRs, fixed per-lane offset
    const uint64_t b0 = sgpr_ptr(base + (size_t)(j0 + wv * RPI) * ld);
    const uint64_t step = (uint64_t)(NW * RPI) * ld * 2;
    const uint32_t m00 = __builtin_amdgcn_readfirstlane(lds + (uint32_t)(wv * RPI * D * 2));
#pragma unroll
    for (int n = 0; n < NI / NW; ++n) {
      const uint64_t rowp = b0 + n * step;
      const uint32_t m0v = m00 + (uint32_t)(n * NW * RPI * D * 2);
      asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
                   :
                   : "s"(m0v), "v"(loff), "s"(rowp)
                   : "memory", "m0");
    }
  } else {
    // tail tile: rows past Tn - 1 repeat row Tn - 1
#pragma unroll
    for (int i0 = 0; i0 < NI; i0 += NW) {
      const int i = i0 + wv;
      const int r = i * RPI + l / CPR;
      const int q = (l % CPR) ^ chunk_swz<D, KIND>(r);
      const int gr = min(j0 + r, Tn - 1);
      const uint32_t off = (uint32_t)((size_t)gr * ld * 2 + 16 * q);
      const uint32_t m0v = __builtin_amdgcn_readfirstlane(lds + (uint32_t)(i * RPI * D * 2));
      asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
                   :
                   : "s"(m0v), "v"(off), "s"(sgpr_ptr(base))
                   : "memory", "m0");
    }
  }
}

// Vector-memory counter wait of step c of a ring pipeline: NS stages of OPS
// loads were issued up front, and every step then issued STO stores and the
// OPS loads of a new stage.  Operations complete in issue order, so this
// waits exactly for the loads of stage c.
// Slot-state registers of a scan wave (16 columns j0 + 4 g + r of slots
// i = 16 nb + cc): the initial states s0k / s0v [unit][m][d] (fp32), or zero
// when they are null; padded slots i >= m are zero.
template <int NB>
__device__ __forceinline__ void init_slot_state(floatx4 (&SK)[NB], floatx4 (&SV)[NB], const float* s0k,
                                                const float* s0v, int unit, int m, int d, int j0, int g, int cc) {
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    SK[nb] = SV[nb] = zero4();
    const int i = 16 * nb + cc;
    if (s0k && i < m) {
      const size_t e = ((size_t)unit * m + i) * d + j0 + 4 * g;
      SK[nb] = *reinterpret_cast<const floatx4*>(s0k + e);
      SV[nb] = *reinterpret_cast<const floatx4*>(s0v + e);
    }
  }
}

// The same registers out to ds0k / ds0v [unit][m][d] (fp32) when not null.
template <int NB>
__device__ __forceinline__ void store_slot_state(const floatx4 (&SK)[NB], const floatx4 (&SV)[NB], float* ok,
                                                 float* ov, int unit, int m, int d, int j0, int g, int cc) {
  if (!ok) return;
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int i = 16 * nb + cc;
    if (i < m) {
      const size_t e = ((size_t)unit * m + i) * d + j0 + 4 * g;
      *reinterpret_cast<floatx4*>(ok + e) = SK[nb];
      *reinterpret_cast<floatx4*>(ov + e) = SV[nb];
    }
  }
}

template <int N>
__device__ __forceinline__ void vm_wait() {
  static_assert(N >= 0 && N < 64, "vmcnt field");
  asm volatile("s_waitcnt vmcnt(%0)" ::"i"(N) : "memory");
}
template <int NS, int OPS, int STO>
__device__ __forceinline__ void vm_wait_steps(int c) {
  static_assert(NS >= 2 && NS <= 4, "ring depth");
  if (c >= NS - 1) {
    vm_wait<(NS - 1) * (OPS + STO)>();
  } else if (c == 0) {
    vm_wait<(NS - 1) * OPS>();
  } else if (c == 1) {
    vm_wait<(NS - 1) * OPS + STO>();
  } else {
    vm_wait<(NS - 1) * OPS + 2 * STO>();
  }
}
