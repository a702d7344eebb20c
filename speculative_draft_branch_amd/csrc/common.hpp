// Device-side helpers shared by the gfx950 kernels: the metadata view, vector
// types, MFMA wrappers, LDS swizzle and wave-level reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

#include "plan.hpp"

namespace ba {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Kernel-visible view of the plan metadata (pointers into the workspace).
struct Meta {
  const int32_t *group_heads;
  const QTile *qtiles;
  const int32_t *fwd_order;
  const int32_t *fwd_pairs;
  const int32_t *fwd_triples;
  const int32_t *tile_row_id;
  const int32_t *tile_row_end;
  const int32_t *row_lo;
  const int32_t *row_hi;
  const int32_t *cu_branch;
  const int32_t *mode;
  const KTile *ktiles;
  const int32_t *bwd_order;
  const int32_t *vt_tiles;
  const int32_t *vt_base;
  const int32_t *brow_lo;
  const int32_t *brow_hi;
  const int32_t *fwd_pair_bk;
  const int32_t *fwd_triple_bk;
  const int32_t *fwd_unit_bt;
  const int32_t *vbt_start;
  // Work counters (zeroed before the launch), one per kv head, or null: the
  // forward / dQ kernel (queue_units) and the dK/dV kernel (queue_ktiles) then
  // take their items by block index instead.
  int *queue_units;
  int *queue_ktiles;
  int64_t N, Nq, Rb, A;
  int32_t hq, hkv, G, d, rows_per_tile;
  int32_t n_qtiles, n_ktiles, n_fwd_pairs, n_vt_tiles, n_fwd_triples, n_vbt_tiles;
  int32_t max_branch;  // longest branch (rows of one anchor)
  float scale;
};

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16 x) { return (float)x; }
template <class T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float x) { return (bf16)x; }

// Tile descriptors are the same for every lane; reading them through
// readfirstlane keeps tile-level control and addressing in scalar registers.
__device__ __forceinline__ int uni(int x) { return __builtin_amdgcn_readfirstlane(x); }

// Work assignment across the XCDs. Items are (index, kv head), numbered index *
// hkv + head, each head's indices in longest-first order; block index b stands
// for item b, so the hardware's round-robin of workgroups over the eight XCDs
// gives each XCD one kv head (its K/V stream through that XCD's L2). The XCDs
// do not run at one speed, though (identical heads finished up to 6% apart), so
// with a counter per head a workgroup takes the next index of its XCD's own
// head and, once that head is done, of any other head: the XCDs then finish
// together. Returns the item, or -1 when every head is done (the workgroup has
// nothing to do). One thread calls it; `counters` holds hkv ints, zeroed before
// the launch.
__device__ __forceinline__ int take_item(int *counters, int n, int hkv) {
  const int xcc = (int)__builtin_amdgcn_s_getreg(20 | (0 << 6) | (3 << 11));  // XCC_ID[3:0]
  for (int h = hkv >= 8 ? xcc : xcc % hkv; h < hkv; h += 8) {
    const int i = atomicAdd(counters + h, 1);
    if (i < n) return i * hkv + h;
  }
  for (int h = 0; h < hkv; ++h) {
    const int i = atomicAdd(counters + h, 1);
    if (i < n) return i * hkv + h;
  }
  return -1;
}

// Workgroups to launch for `items` items of a kernel that takes one item per
// workgroup: with counters an eighth more (at least 8), since each XCD is dealt
// a fixed share of the workgroups and one that runs ahead needs spare ones to
// take over items of the others' heads; the spares that find every head done
// end at once. Without counters, one workgroup per item.
inline unsigned queue_grid(int64_t items, const int *counters) {
  return (unsigned)(counters ? items + (items / 8 > 8 ? items / 8 : 8) : items);
}

// Workgroups to launch for a kernel whose workgroups loop over items while
// the counters last (the d = 128 forward): one per compute unit of the current
// device (that kernel fits one workgroup per compute unit), at most one per
// item; without counters, one per item.
unsigned persistent_grid(int64_t items, const int *counters);

// take_item for the whole workgroup (slot: a __shared__ int); counters null:
// the block index.
__device__ __forceinline__ int workgroup_item(int *counters, int n, int hkv, int *slot) {
  if (!counters) return (int)blockIdx.x;
  if (threadIdx.x == 0) *slot = take_item(counters, n, hkv);
  __syncthreads();
  return *slot;
}
__device__ __forceinline__ QTile load_qtile(const QTile *p) {
  QTile t = *p;
  t.row_begin = uni(t.row_begin);
  t.nrows = uni(t.nrows);
  t.kv_lo = uni(t.kv_lo);
  t.end_min = uni(t.end_min);
  t.end_max = uni(t.end_max);
  t.seq = uni(t.seq);
  return t;
}
__device__ __forceinline__ KTile load_ktile(const KTile *p) {
  KTile t = *p;
  t.key_lo = uni(t.key_lo);
  t.key_hi = uni(t.key_hi);
  t.qt_begin = uni(t.qt_begin);
  t.qt_end = uni(t.qt_end);
  return t;
}

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Swap the two 32-lane halves of a wave: returns the value held by lane ^ 32.
__device__ __forceinline__ float half_swap(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float((threadIdx.x & 32) ? r[0] : r[1]);
}
// max / sum of a value over the two lanes l and l ^ 32.
__device__ __forceinline__ float half_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float half_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ int wave_min(int x) {
  for (int o = 32; o >= 1; o >>= 1) x = min(x, __shfl_xor(x, o, 64));
  return x;
}
__device__ __forceinline__ int wave_max(int x) {
  for (int o = 32; o >= 1; o >>= 1) x = max(x, __shfl_xor(x, o, 64));
  return x;
}

// LDS tiles of key rows (HD bf16 each: 256-byte rows at HD = 128, 128-byte rows
// for HD = 64 and for the 64-key V^T tiles) are stored in 16-byte chunks whose
// index is XOR-swizzled by the row, so that the row-wise 16-byte operand reads
// (16 rows at one chunk) and the transposing reads (4 rows x 4 chunks) spread
// over the 64 banks. A 128-byte row shares its bank line with the next row, so
// its swizzle is a bijection of row bits 1-3 (even and odd rows each get eight
// distinct chunks), with bit 2 following row bit 1 for the transposing reads;
// the bank counters read zero conflicts for both patterns with it.
template <int HD>
__device__ __forceinline__ int swz(int row) {
  if constexpr (HD == 128) return ((row & 7) << 1) | ((row >> 3) & 1);
  else return (((row >> 1) & 1) << 2) | (((row >> 2) & 1) << 1) | ((row >> 3) & 1);
}
template <int HD>
__device__ __forceinline__ int lds_off(int row, int d) {  // element offset of (row, d)
  return row * HD + ((((d >> 3) ^ swz<HD>(row))) << 3) + (d & 7);
}

// LDS DMA (global_load_lds: each lane's BYTES land at lds_dst + lane * BYTES,
// lds_dst wave-uniform) issued from inline asm, so that the compiler's
// wait-count tracking does not see it. Seeing one, hipcc treats every later LDS
// read in the loop as unordered and waits for all LDS reads in flight
// (lgkmcnt(0)) before the first use of any of them, which turns each operand
// pipeline into batches. Every reader of DMA'd data waits through dma_barrier
// (a vmcnt wait and a workgroup barrier, both visible to the compiler); an
// untracked load only makes the compiler's own vmcnt waits more conservative.
// The memory clobber keeps every LDS access on its side of the request.
template <int BYTES>
__device__ __forceinline__ void lds_dma(const void *src, const void *lds_dst) {
  static_assert(BYTES == 4 || BYTES == 16, "dword or dwordx4");
  // the LDS offset is the low half of a generic pointer into LDS
  const uint32_t m0 = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(uintptr_t)lds_dst);
  if constexpr (BYTES == 16)
    asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off" : : "v"(src), "{m0}"(m0)
                 : "memory");
  else
    asm volatile("s_nop 0\n\tglobal_load_lds_dword %0, off" : : "v"(src), "{m0}"(m0)
                 : "memory");
}

// Padded LDS tiles: each row of HD bf16 followed by 48 unused bytes (19 four-
// bank groups per row at d = 128, an odd count). Sixteen consecutive rows at
// the same column then start in sixteen different 4-bank groups, so operand
// reads need no swizzle and every operand's address is a per-lane base plus a
// constant (no address arithmetic per read). Measured against 16 and 32 bytes
// of padding, 48 gave the fewest bank conflicts over the two read patterns. A
// row is written by one LDS DMA instruction, 4 bytes per lane (HD / 2 lanes).
template <int HD>
constexpr int kPadRowBytes = HD * 2 + 48;

// Rows [0, ROWS) of a contiguous [rows][HD] bf16 source into a padded LDS tile;
// rows r with r % NW == w are this wave's. Asynchronous (vmcnt).
template <int HD, int ROWS, int NW>
__device__ __forceinline__ void stage_padded_async(bf16 *lds, const bf16 *__restrict__ src, int wave, int lane) {
  static_assert(ROWS % NW == 0, "rows per wave");
  constexpr int LANES = HD / 2;  // 4-byte lanes per row
  const int w = uni(wave);  // row choice, hence both addresses' row parts, is wave-uniform
  const uint32_t lane_off = (uint32_t)lane * 4u;
#pragma unroll
  for (int it = 0; it < ROWS / NW; ++it) {
    const int r = it * NW + w;
    const char *row = reinterpret_cast<const char *>(src + (int64_t)r * HD);
    if (LANES == 64 || lane < LANES)
      lds_dma<4>(row + lane_off, reinterpret_cast<char *>(lds) + r * kPadRowBytes<HD>);
  }
}
// Row read (A operand with k = column): lane reads row 32*blk + lane%32,
// columns 16*ks + 8*(lane/32) .. +7.
template <int HD>
__device__ __forceinline__ uint32_t pad_row_base(int lane) {
  return (uint32_t)((lane & 31) * kPadRowBytes<HD> + (lane >> 5) * 16);
}
template <int HD>
__device__ __forceinline__ bf16x8 pad_row_read(const bf16 *tile, uint32_t base, int blk, int ks) {
  return *reinterpret_cast<const bf16x8 *>(reinterpret_cast<const char *>(tile) + base +
                                           blk * 32 * kPadRowBytes<HD> + ks * 32);
}
// The same two reads from a 32-bit LDS address `a` (tile, lane offset and any
// row-block offset already added), plus an immediate offset.
template <int HD>
__device__ __forceinline__ bf16x8 pad_row_read_at(uint32_t a, int ks) {
  return *(const __attribute__((address_space(3))) bf16x8 *)(uintptr_t)(a + ks * 32);
}
template <int HD>
__device__ __forceinline__ i16x4 pad_tr_read_at(uint32_t a, int c, int kk, int dt) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) i16x4 *)(uintptr_t)(a + (16 * kk + 8 * c) * kPadRowBytes<HD> + dt * 64));
}
// Transposing read (operand with k = row): the 16-lane group g = lane/16 reads
// rows 16*kk + 4*(g/2) + (lane%16)/4 + 8c, columns 32*dt + 16*(g%2) + 4*(lane%4) .. +3.
template <int HD>
__device__ __forceinline__ uint32_t pad_tr_base(int lane) {
  const int g = lane >> 4, in_j = (lane & 15) >> 2, in_q = lane & 3;
  return (uint32_t)((4 * (g >> 1) + in_j) * kPadRowBytes<HD> + (16 * (g & 1) + 4 * in_q) * 2);
}
template <int HD>
__device__ __forceinline__ i16x4 pad_tr_read(const bf16 *tile, uint32_t base, int c, int kk, int dt) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4 *)(
      reinterpret_cast<const char *>(tile) + base + (16 * kk + 8 * c) * kPadRowBytes<HD> + dt * 64));
}

// Per-lane addressing of MFMA operand reads from a swizzled [row][HD] bf16 LDS
// tile. The swizzle XORs chunk-index bits that the k-step (or d-block) index
// and the lane's own chunk bits never share, so an operand's byte offset is
// (step << c) ^ t plus a per-lane row base.
//
// Row read (ds_read_b128, A operand with k = d): lane reads row
// 32*blk + r (r = lane % 32 plus a caller offset), chunk 2*ks + lane/32, at
// byte base + ((ks << 5) ^ t) + blk * 32 * HD * 2 (the forward keeps the first
// two terms per ks in registers, so a read is a register plus an immediate).
template <int HD>
__device__ __forceinline__ void row_read_init(int r, int lane, uint32_t &base, uint32_t &t) {
  base = (uint32_t)(r * HD * 2);
  t = (uint32_t)((lane >> 5) ^ swz<HD>(r)) << 4;
}
// Transposing read (ds_read_b64_tr_b16, operand with k = row): the 16-lane
// group g = lane/16 reads rows 16*kk + 4*(g/2) + (lane%16)/4 + 8c, d = 32*dt +
// 16*(g%2) + 4*(lane%4) .. +3; one (base, t) pair per c.
template <int HD>
__device__ __forceinline__ void tr_read_init(int lane, int c, uint32_t &base, uint32_t &t) {
  const int g = lane >> 4, in_j = (lane & 15) >> 2, in_q = lane & 3;
  const int row = 4 * (g >> 1) + in_j + 8 * c;
  const int cl = (g & 1) * 2 + (in_q >> 1);  // chunk within a 32-wide d block
  base = (uint32_t)(row * HD * 2 + 8 * (in_q & 1));
  t = (uint32_t)(cl ^ swz<HD>(row)) << 4;
}

// Transposed LDS read (gfx950 ds_read_b64_tr_b16): within each 16-lane group,
// output lane i, slot j takes element (i % 4) of the 8 bytes addressed by input
// lane 4j + i/4.
__device__ __forceinline__ i16x4 lds_read_tr(const bf16 *p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4 *)(p));
}
template <int HD>
__device__ __forceinline__ i16x4 tr_read(const bf16 *tile, uint32_t base, uint32_t t, int kk, int dt) {
  const uint32_t off = base + (((uint32_t)dt << 6) ^ t) + (uint32_t)(kk * 16 * HD * 2);
  return lds_read_tr(reinterpret_cast<const bf16 *>(reinterpret_cast<const char *>(tile) + off));
}
// Makes the compiler treat a per-lane address term as freshly produced, so the
// addresses derived from it are recomputed where they are used (one VALU op per
// read) rather than hoisted into one live register per read.
__device__ __forceinline__ void opaque(uint32_t &x) { asm volatile("" : "+v"(x)); }
// The lane id, recomputed where it is used (two VALU ops) instead of living in
// a register across a loop; the compiler cannot hoist or spill it.
__device__ __forceinline__ int lane_id_here() {
  int l;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
  return l;
}

// Stage rows [k0, k0 + ROWS) of a [rows, Hkv, HD] bf16 tensor (kv head g) into
// an LDS tile in the swizzled layout; rows past `last` (inclusive bound) are
// zero-filled. All NT threads of the block take part.
template <int HD, int ROWS, int NT>
__device__ __forceinline__ void stage_rows(bf16 *lds, const bf16 *__restrict__ src, int hkv, int g, int k0, int last,
                                           int tid) {
  constexpr int NCH = HD / 8;
  static_assert((ROWS * NCH) % NT == 0, "tile must split evenly over the block");
#pragma unroll
  for (int it = 0; it < ROWS * NCH / NT; ++it) {
    const int c = tid + it * NT;
    const int r = c / NCH, ch = c % NCH;
    const int key = k0 + r;
    uint4 x = {0u, 0u, 0u, 0u};
    if (key <= last) x = *reinterpret_cast<const uint4 *>(src + ((int64_t)key * hkv + g) * HD + ch * 8);
    *reinterpret_cast<uint4 *>(lds + r * HD + ((ch ^ swz<HD>(r)) << 3)) = x;
  }
}

// Asynchronous staging of a [ROWS x HD] bf16 tile into LDS with global_load_lds
// (16 bytes per lane, gfx950): each wave's 1 KB block of the swizzled tile is
// written straight into LDS, lane l of block b fetching the logical chunk that
// the swizzle places at LDS offset b*1KB + 16*l. Completion is tracked by
// vmcnt: dma_barrier() before the tile is read.
//
// The per-lane part of each address (row within the tile, chunk) is fixed for
// the kernel's life, so it is computed once; a tile only moves the uniform base.
template <int HD, int ROWS, int NT>
struct AsyncTile {
  static constexpr int NCH = HD / 8;         // 16-byte chunks per row
  static constexpr int RPB = 64 / NCH;       // rows per 1 KB wave block
  static constexpr int BLOCKS = ROWS / RPB;  // 1 KB blocks in the tile
  static_assert(BLOCKS % (NT / 64) == 0, "tile must split evenly over the waves");
  static constexpr int PER_WAVE = BLOCKS / (NT / 64);
  int row[PER_WAVE];        // tile row of this lane's chunk in each of its wave's blocks
  uint32_t off[PER_WAVE];   // byte offset of that chunk from the tile's first row
  int lds_block;            // first 1 KB block of this wave (wave-uniform)
  int row_stride;           // elements between consecutive rows in global memory

  __device__ __forceinline__ void init(int row_stride_elems, int tid) {
    const int lane = tid & 63;
    row_stride = row_stride_elems;
    lds_block = uni(tid >> 6) * PER_WAVE;
#pragma unroll
    for (int it = 0; it < PER_WAVE; ++it) {
      const int r = (lds_block + it) * RPB + lane / NCH;
      row[it] = r;
      off[it] = (uint32_t)(r * row_stride_elems + (((lane % NCH) ^ swz<HD>(r)) << 3)) * 2u;
    }
  }
  // Tile rows [k0, k0 + ROWS) from `base` (pointer to row 0 of the tensor,
  // already offset to the kv head); rows past `last` are clamped to `last`.
  __device__ __forceinline__ void load(bf16 *lds, const bf16 *__restrict__ base, int k0, int last) const {
    const char *tb = reinterpret_cast<const char *>(base + (int64_t)k0 * row_stride);
    if (k0 + ROWS - 1 <= last) {
#pragma unroll
      for (int it = 0; it < PER_WAVE; ++it)
        lds_dma<16>(tb + off[it], lds + (lds_block + it) * 512);
    } else {
#pragma unroll
      for (int it = 0; it < PER_WAVE; ++it) {
        // rows past the end read row `last` instead (callers mask those keys)
        const uint32_t back = (uint32_t)max(k0 + row[it] - last, 0) * (uint32_t)row_stride * 2u;
        lds_dma<16>(tb + (off[it] - back), lds + (lds_block + it) * 512);
      }
    }
  }
  // As load(), for a tile that may also begin before row `first` (k0 may be
  // negative): rows outside [first, last] read the nearer of the two.
  __device__ __forceinline__ void load_window(bf16 *lds, const bf16 *__restrict__ base, int k0, int first,
                                              int last) const {
    if (k0 >= first) {
      load(lds, base, k0, last);
      return;
    }
    const char *b = reinterpret_cast<const char *>(base);
#pragma unroll
    for (int it = 0; it < PER_WAVE; ++it) {
      const int r = min(max(k0 + row[it], first), last);
      const uint32_t chunk = off[it] - (uint32_t)(row[it] * row_stride) * 2u;  // byte offset within the row
      lds_dma<16>(b + (int64_t)r * row_stride * 2 + chunk, lds + (lds_block + it) * 512);
    }
  }
};

template <int HD, int ROWS, int NT>
__device__ __forceinline__ void stage_rows_async(bf16 *lds, const bf16 *__restrict__ src, int hkv, int g, int k0,
                                                 int last, int tid) {
  AsyncTile<HD, ROWS, NT> t;
  t.init(hkv * HD, tid);
  t.load(lds, src + (int64_t)g * HD, k0, last);
}

// Asynchronous copy of 64*n consecutive 32-bit words into LDS by one wave
// (global_load_lds, 4 bytes per lane).
template <int N>
__device__ __forceinline__ void stage_words_async(void *lds, const void *__restrict__ src, int lane) {
#pragma unroll
  for (int it = 0; it < N; ++it)
    lds_dma<4>(static_cast<const uint32_t *>(src) + it * 64 + lane, static_cast<uint32_t *>(lds) + it * 64);
}

// Workgroup barrier after this wave's LDS reads and all but its VM most recent
// vector-memory requests (LDS DMA among them) have completed: every tile
// requested before those is in LDS for every wave after the barrier, and no
// LDS read of the phase before it is still in flight. This barrier is the only
// wait for DMA'd data (lds_dma hides the DMA from the compiler's tracking); the
// wait goes through the builtin so the compiler's own wait insertion sees it.
// The empty asm statements stop the compiler moving memory accesses across.
// VM = 63 waits for LDS reads only.
template <int VM>
__device__ __forceinline__ void dma_barrier() {
  static_assert(VM >= 0 && VM <= 63, "vmcnt field");
  asm volatile("" ::: "memory");
  // s_waitcnt fields: vmcnt [3:0] and [15:14], expcnt [6:4], lgkmcnt [11:8]
  __builtin_amdgcn_s_waitcnt((VM & 15) | ((VM >> 4) << 14) | 0x0070);
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

__device__ __forceinline__ bf16x8 join(i16x4 a, i16x4 b) {
  typedef short i16x8 __attribute__((ext_vector_type(8)));
  i16x8 r = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  return __builtin_bit_cast(bf16x8, r);
}

}  // namespace ba
