// Landmark pooling: Kbar[b,g,blk,:] = mean of K[b,g,blk*L .. blk*L+L-1,:]
// and the same for V (the landmark tokens of the page "Scaling GPU Cluster
// for Million Token Context", section "Why Sparse Attention Changes the
// Game", taken as block means).  Pure streaming: every input byte is read
// once with 16-byte loads; float32 accumulation in a fixed order, so the
// result is deterministic; round-to-nearest-even into the input dtype.
//
// Append (incremental decode): one new K/V row per sequence is stored and,
// when it completes a landmark block, that block is pooled again by the
// same code, so a cache filled token by token holds the same landmark bits
// as one pooled at once.
#include "msa_device.hpp"
#include "msa_internal.hpp"

namespace msa {
namespace {

template <typename T>
struct Chunk;  // one 16-byte load

template <>
struct Chunk<uint16_t> {
  static constexpr int kElems = 8;
  __device__ static void add(float* acc, const u32x4& v) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc[2 * e] += bf16_bits_to_f32(v[e] & 0xffffu);
      acc[2 * e + 1] += bf16_bits_to_f32(v[e] >> 16);
    }
  }
  __device__ static void store(uint16_t* dst, const float* vals) {
    u32x4 o;
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] = pack_bf16x2(vals[2 * e], vals[2 * e + 1]);
    *reinterpret_cast<u32x4*>(dst) = o;
  }
};

template <>
struct Chunk<float> {
  static constexpr int kElems = 4;
  __device__ static void add(float* acc, const u32x4& v) {
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[e] += __uint_as_float(v[e]);
  }
  __device__ static void store(float* dst, const float* vals) {
    *reinterpret_cast<f32x4*>(dst) = f32x4{vals[0], vals[1], vals[2], vals[3]};
  }
};

template <typename T, int D>
struct PoolShape {
  static constexpr int kE = Chunk<T>::kElems;
  static constexpr int kChunks = D / kE;
  static constexpr int kRowLanes = 256 / kChunks;
};

// Rows of one block: consecutive rows from base, or rows row0 + r of a
// paged cache looked up in a block table (an invalid page id reads page 0).
template <typename T, int D>
struct RowsContig {
  const T* base;
  __device__ __forceinline__ const T* row(int r) const { return base + (size_t)r * D; }
};

template <int D>
struct RowsPaged {
  const uint16_t* pool;  // this KV head's rows of physical page 0
  const int32_t* tbl;    // this sequence's block table
  size_t pstride;        // elements between consecutive physical pages of the KV head
  int row0, shift, max_pages, num_pages;
  __device__ __forceinline__ const uint16_t* row(int r) const {
    const int g = row0 + r;
    int id = tbl[min(g >> shift, max_pages - 1)];
    id = (unsigned)id < (unsigned)num_pages ? id : 0;
    return pool + (size_t)id * pstride + (size_t)(g & ((1 << shift) - 1)) * D;
  }
};

// Mean of the L rows of one block (row stride D elements) by one workgroup
// of 256 threads, laid out as kRowLanes row lanes x kChunks 16-byte column
// chunks.  Row lane rl sums rows rl, rl + kRowLanes, ... of the block in
// ascending order, issuing the loads of up to 16 of its rows before adding
// any; the row lanes of each wavefront are then combined by a butterfly of
// lane exchanges (both partners of an exchange form the same sum, addition
// being commutative), the 4 wavefronts' sums are added in order through
// LDS, and the total is divided by L.  The order is fixed, so the result is
// deterministic.  With LAST, row L-1 is read from `last` instead of the
// block (the row an append is writing), which gives the same bits as
// pooling the block once that row is stored.  Called by every thread.
template <typename T, int D, bool LAST, typename Rows>
__device__ __forceinline__ void pool_block(const Rows& rows, const T* __restrict__ last, int L, T* __restrict__ dst,
                                           float (*red)[D]) {
  using PS = PoolShape<T, D>;
  constexpr int kE = PS::kE, kChunks = PS::kChunks, kRowLanes = PS::kRowLanes;
  constexpr int kBatch = 16;
  static_assert(kChunks <= 64 && 64 % kChunks == 0, "a wavefront holds whole rows of chunks");
  const int ch = threadIdx.x % kChunks;
  const int rl = threadIdx.x / kChunks;
  float acc[kE];
#pragma unroll
  for (int e = 0; e < kE; ++e) acc[e] = 0.f;

  const u32x4* lp = reinterpret_cast<const u32x4*>(last) + ch;
  auto row = [&](int r) -> const u32x4* {
    return (LAST && r == L - 1) ? lp : reinterpret_cast<const u32x4*>(rows.row(r)) + ch;
  };
  int r = rl;
  for (; r + (kBatch - 1) * kRowLanes < L; r += kBatch * kRowLanes) {
    u32x4 v[kBatch];
#pragma unroll
    for (int i = 0; i < kBatch; ++i) v[i] = *row(r + i * kRowLanes);
#pragma unroll
    for (int i = 0; i < kBatch; ++i) Chunk<T>::add(acc, v[i]);
  }
  for (; r + 3 * kRowLanes < L; r += 4 * kRowLanes) {
    const u32x4 a = *row(r);
    const u32x4 b = *row(r + kRowLanes);
    const u32x4 c = *row(r + 2 * kRowLanes);
    const u32x4 d = *row(r + 3 * kRowLanes);
    Chunk<T>::add(acc, a);
    Chunk<T>::add(acc, b);
    Chunk<T>::add(acc, c);
    Chunk<T>::add(acc, d);
  }
  for (; r < L; r += kRowLanes) Chunk<T>::add(acc, *row(r));

  // lanes l and l ^ (kChunks << k) hold the same chunk of other rows
#pragma unroll
  for (int off = kChunks; off < 64; off <<= 1) {
#pragma unroll
    for (int e = 0; e < kE; ++e) acc[e] += __shfl_xor(acc[e], off);
  }
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) < kChunks) {
#pragma unroll
    for (int e = 0; e < kE; ++e) red[wave][ch * kE + e] = acc[e];
  }
  __syncthreads();
  if (threadIdx.x < kChunks) {
    float out[kE];
#pragma unroll
    for (int e = 0; e < kE; ++e) {
      const int c = threadIdx.x * kE + e;
      out[e] = (((red[0][c] + red[1][c]) + red[2][c]) + red[3][c]) / (float)L;
    }
    Chunk<T>::store(dst + threadIdx.x * kE, out);
  }
}

// One workgroup per (tensor, batch*kv_head, landmark).
template <typename T, int D>
__global__ __launch_bounds__(256) void pool_kernel(const T* __restrict__ K, const T* __restrict__ V,
                                                   T* __restrict__ Kbar, T* __restrict__ Vbar, int n,
                                                   int G, int L, int blocks_per_tensor) {
  __shared__ float red[4][D];
  const int wg = blockIdx.x;
  const bool is_v = wg >= blocks_per_tensor;
  const int blk = is_v ? wg - blocks_per_tensor : wg;  // over batch*kv_heads*G
  const int bh = blk / G;
  const int lm = blk - bh * G;
  const T* src = (is_v ? V : K) + ((size_t)bh * n + (size_t)lm * L) * D;
  T* dst = (is_v ? Vbar : Kbar) + (size_t)blk * D;
  pool_block<T, D, false>(RowsContig<T, D>{src}, nullptr, L, dst, red);
}

// Append: one workgroup per (tensor, batch*kv_head).  The sequence's new
// row goes to position pos of its cache; if it is the last row of block
// blk = (pos+1)/L - 1, that block's landmark is pooled again (rows before
// pos from the cache, row pos from the new token).  A position outside
// [0, C) leaves the sequence untouched.
//
// Paged caches (table != null): pools [num_pages][Hkv][page][D]; row pos of
// sequence b lives at row pos mod page of physical page table[b][pos/page].
// A sequence whose page id for pos lies outside [0, num_pages) is left
// untouched (nothing is written); rows of the pooled block are looked up
// one by one.
struct AppendArgs {
  const int32_t* positions;
  const uint16_t *k_new, *v_new;
  uint16_t *Kc, *Vc, *Kbar, *Vbar;
  int Hkv, C, G, L, pairs;
  const int32_t* table;
  int shift, max_pages, num_pages;
};

template <int D>
__global__ __launch_bounds__(256) void append_kernel(AppendArgs A) {
  __shared__ float red[4][D];
  const int wg = blockIdx.x;
  const bool is_v = wg >= A.pairs;
  const int bk = is_v ? wg - A.pairs : wg;  // b * Hkv + kvh
  const int b = bk / A.Hkv, kvh = bk % A.Hkv;
  const int pos = A.positions[b];
  if (pos < 0 || pos >= A.C) return;
  const uint16_t* src = (is_v ? A.v_new : A.k_new) + (size_t)bk * D;
  uint16_t* dst_row;
  RowsPaged<D> paged{};
  if (A.table != nullptr) {
    const size_t page_elems = (size_t)D << A.shift;
    paged = RowsPaged<D>{(is_v ? A.Vc : A.Kc) + (size_t)kvh * page_elems, A.table + (size_t)b * A.max_pages,
                         (size_t)A.Hkv * page_elems, 0, A.shift, A.max_pages, A.num_pages};
    const int id = paged.tbl[pos >> A.shift];
    if ((unsigned)id >= (unsigned)A.num_pages) return;
    dst_row = const_cast<uint16_t*>(paged.pool) + (size_t)id * paged.pstride +
              (size_t)(pos & ((1 << A.shift) - 1)) * D;
  } else {
    dst_row = (is_v ? A.Vc : A.Kc) + ((size_t)bk * A.C + pos) * D;
  }
  if (threadIdx.x < D / 8) {
    reinterpret_cast<u32x4*>(dst_row)[threadIdx.x] = reinterpret_cast<const u32x4*>(src)[threadIdx.x];
  }
  if (A.G > 0 && (pos + 1) % A.L == 0) {
    const int blk = (pos + 1) / A.L - 1;
    uint16_t* dst = (is_v ? A.Vbar : A.Kbar) + ((size_t)bk * A.G + blk) * D;
    if (A.table != nullptr) {
      paged.row0 = blk * A.L;
      pool_block<uint16_t, D, true>(paged, src, A.L, dst, red);
    } else {
      const uint16_t* cache = (is_v ? A.Vc : A.Kc) + (size_t)bk * A.C * D;
      pool_block<uint16_t, D, true>(RowsContig<uint16_t, D>{cache + (size_t)blk * A.L * D}, src, A.L, dst, red);
    }
  }
}

template <typename T, int D>
hipError_t launch_pool_t(const msa_attn_desc& d, const void* K, const void* V, void* Kb, void* Vb,
                         hipStream_t stream) {
  const int G = d.num_landmarks;
  const int L = d.seq_len / G;
  const int per = d.batch * d.heads_kv * G;
  hipLaunchKernelGGL((pool_kernel<T, D>), dim3(2 * per), dim3(256), 0, stream,
                     static_cast<const T*>(K), static_cast<const T*>(V), static_cast<T*>(Kb),
                     static_cast<T*>(Vb), d.seq_len, G, L, per);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_append(const msa_decode_desc& d, const int32_t* positions, const DecodePaging* paging,
                         const void* k_new, const void* v_new, void* Kc, void* Vc, void* Kbar, void* Vbar,
                         hipStream_t stream) {
  const int G = d.num_landmarks;
  AppendArgs A{positions, static_cast<const uint16_t*>(k_new), static_cast<const uint16_t*>(v_new),
               static_cast<uint16_t*>(Kc), static_cast<uint16_t*>(Vc), static_cast<uint16_t*>(Kbar),
               static_cast<uint16_t*>(Vbar), d.heads_kv, d.ctx_len, G, G > 0 ? d.ctx_len / G : 1,
               d.batch * d.heads_kv, nullptr, 0, 0, 0};
  if (paging != nullptr) {
    A.table = paging->table;
    A.shift = paging->page_shift;
    A.max_pages = paging->max_pages;
    A.num_pages = paging->num_pages;
  }
  if (d.head_dim == 128) {
    hipLaunchKernelGGL((append_kernel<128>), dim3(2 * A.pairs), dim3(256), 0, stream, A);
  } else {
    hipLaunchKernelGGL((append_kernel<64>), dim3(2 * A.pairs), dim3(256), 0, stream, A);
  }
  return hipGetLastError();
}

hipError_t launch_pool(const msa_attn_desc& d, const void* K, const void* V, void* Kbar, void* Vbar,
                       hipStream_t stream) {
  if (d.in_dtype == MSA_DTYPE_BF16) {
    return d.head_dim == 128 ? launch_pool_t<uint16_t, 128>(d, K, V, Kbar, Vbar, stream)
                             : launch_pool_t<uint16_t, 64>(d, K, V, Kbar, Vbar, stream);
  }
  return d.head_dim == 128 ? launch_pool_t<float, 128>(d, K, V, Kbar, Vbar, stream)
                           : launch_pool_t<float, 64>(d, K, V, Kbar, Vbar, stream);
}

}  // namespace msa
