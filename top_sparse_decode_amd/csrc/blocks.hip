// Block-compressed QSA selection ("QSA cache sharding": the compressed cache
// and the top-k over compressed blocks; "Context parallelism for QSA
// attention and the sparse indexer": block compression of the raw index-K
// before scoring). Blocks of Bs consecutive tokens get one compressed FP8
// index key each, kept in a paged pool of its own; the decode step scores
// and selects blocks with the token kernels, and the selected blocks are
// expanded to their tokens for the attention.
//
// index_k_compress: one wave per page of tokens. Block sizes are powers of
// two up to 64, so a block never crosses a token page and the blocks of one
// token page share one compressed page: one page-id load each. Lane group
// s = lane / 8 holds tokens 8s .. 8s + 7 of the page, 16 dimensions per lane
// (one 16-byte load per token), so a block's tokens sit in one lane group
// (Bs <= 8) or in Bs / 8 neighbouring groups combined by lane exchanges.
// The block's key is the mean of its tokens' decoded keys: E4M3 values are
// multiples of 2^-9 below 2^9 in magnitude, so any sum of at most 64 of them
// lies below 2^15 and needs at most 24 significant bits, and the f32 sum is
// exact in any order. A full block divides by a power of two (exact); a
// short last block divides in f64 and rounds once to f32, which equals the
// correctly rounded f32 quotient. The mean is encoded by the gfx950
// converter (nearest, ties to even) after a clamp to +-448.
//
// expand_blocks: one workgroup per row; a block scan of each selected
// block's token count gives its output offset, and each output position
// finds its block by binary search over the offsets, so the token stores
// are contiguous across lanes.
#include "device_common.h"
#include "launch.h"
#include "topk_common.h"

namespace tsd {
namespace {

constexpr int kCW = 4;            // compress waves per workgroup
constexpr int kDi = 128;
constexpr int kXT = 1024;         // expand threads

template <int BS>
__global__ __launch_bounds__(kCW * kWave) void index_k_compress_kernel(
    tsd_compress_args a) {
  constexpr int kT = BS < 8 ? BS : 8;  // a block's tokens in one lane group
  const int b = blockIdx.y;
  const int lane = threadIdx.x & (kWave - 1);
  int64_t n = a.seq_lens[b];
  n = clamp_len(n, a.pt_stride * kPage);
  const int64_t nblk = (n + BS - 1) / BS;
  const int64_t from = a.from_block ? (a.from_block[b] < 0 ? 0 : a.from_block[b]) : 0;
  int64_t jend = from + a.max_blocks < nblk ? from + a.max_blocks : nblk;
  jend = jend < a.cpt_stride * kPage ? jend : a.cpt_stride * kPage;
  // token page of this wave (wave-uniform from here on)
  const int64_t p = from * BS / kPage +
                    static_cast<int64_t>(blockIdx.x) * kCW + (threadIdx.x >> 6);
  if (from >= jend || p * kPage >= jend * BS) return;
  const int32_t page = a.page_table[static_cast<int64_t>(b) * a.pt_stride + p];
  if (page < 0 || page >= a.num_pages) return;
  const int32_t cpage =
      a.cpage_table[static_cast<int64_t>(b) * a.cpt_stride + p * kPage / BS / kPage];
  if (cpage < 0 || cpage >= a.num_cpages) return;
  const int s = lane >> 3;             // tokens 8s .. 8s + 7 of the page
  const int dq = (lane & 7) * 16;      // dimensions dq .. dq + 15
  const int64_t t_grp = p * kPage + s * 8;
  const uint4* src = reinterpret_cast<const uint4*>(
      a.index_k_pool + (static_cast<int64_t>(page) * kPage + s * 8) * kDi + dq);
  uint4 raw[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) raw[i] = src[i * (kDi / 16)];
#pragma unroll
  for (int q = 0; q < 8 / kT; ++q) {
    float acc[16];
#pragma unroll
    for (int d = 0; d < 16; ++d) acc[d] = 0.f;
#pragma unroll
    for (int i = q * kT; i < q * kT + kT; ++i) {
      const bool in = t_grp + i < n;   // slots past the length may hold anything
      const uint32_t w[4] = {raw[i].x, raw[i].y, raw[i].z, raw[i].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float f[4];
        fp8x4_to_f32(w[e], f);
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[e * 4 + c] += in ? f[c] : 0.f;
      }
    }
#pragma unroll
    for (int m = 8; m < BS; m <<= 1)   // neighbouring groups of one block
#pragma unroll
      for (int d = 0; d < 16; ++d) acc[d] += __shfl_xor(acc[d], m);
    const int64_t t0 = t_grp + q * kT;  // first token of the block (leaders)
    const int64_t j = t0 / BS;
    const bool leader = BS <= 8 || (s * 8) % BS == 0;
    if (!leader || j < from || j >= jend) continue;
    const int64_t len = n - t0 < BS ? n - t0 : BS;
    uint32_t out[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float mv[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const float sum = acc[e * 4 + c];
        const float mean = len == BS ? sum * (1.f / BS)
                                     : static_cast<float>(static_cast<double>(sum) /
                                                          static_cast<double>(len));
        mv[c] = fminf(fmaxf(mean, -448.f), 448.f);
      }
      int x = __builtin_amdgcn_cvt_pk_fp8_f32(mv[0], mv[1], 0, false);
      x = __builtin_amdgcn_cvt_pk_fp8_f32(mv[2], mv[3], x, true);
      out[e] = static_cast<uint32_t>(x);
    }
    const int64_t cslot = static_cast<int64_t>(cpage) * kPage + j % kPage;
    *reinterpret_cast<uint4*>(a.ck_pool + cslot * kDi + dq) =
        make_uint4(out[0], out[1], out[2], out[3]);
  }
}

__global__ __launch_bounds__(kXT) void expand_blocks_kernel(
    const int32_t* __restrict__ sel, const int32_t* __restrict__ count,
    int kb, int Bs, const int32_t* __restrict__ row_lens, int kt,
    int32_t* __restrict__ tok, int32_t* __restrict__ tok_count) {
  __shared__ uint32_t off[TSD_MAX_TOPK];  // output offset of selected block i
  __shared__ int32_t blk[TSD_MAX_TOPK];   // its block id
  __shared__ uint32_t lds[kXT / kWave + 1];
  const int row = blockIdx.x;
  const int tid = threadIdx.x;
  const int64_t n = row_lens[row] < 0 ? 0 : row_lens[row];
  int32_t c = count[row];
  c = c < 0 ? 0 : (c > kb ? kb : c);
  // thread t owns selected blocks [4t, 4t + 4)
  constexpr int kPer = TSD_MAX_TOPK / kXT;
  int32_t j[kPer];
  uint32_t len[kPer], sum = 0;
#pragma unroll
  for (int q = 0; q < kPer; ++q) {  // loads issued before count is known
    const int i = tid * kPer + q;
    j[q] = i < kb ? sel[static_cast<int64_t>(row) * kb + i] : -1;
  }
#pragma unroll
  for (int q = 0; q < kPer; ++q) {
    if (tid * kPer + q >= c) j[q] = -1;
    int64_t l = 0;
    if (j[q] >= 0) {
      const int64_t t0 = static_cast<int64_t>(j[q]) * Bs;
      l = t0 + Bs < n ? Bs : n - t0;
      l = l < 0 ? 0 : l;
    }
    len[q] = static_cast<uint32_t>(l);
    sum += len[q];
  }
  uint32_t pos = block_exclusive_scan<kXT>(sum, lds);
  if (tid == kXT - 1) lds[kXT / kWave] = pos + sum;
#pragma unroll
  for (int q = 0; q < kPer; ++q) {
    off[tid * kPer + q] = pos;
    blk[tid * kPer + q] = j[q];
    pos += len[q];
  }
  __syncthreads();
  const uint32_t total = lds[kXT / kWave];
  const uint32_t m = total < static_cast<uint32_t>(kt) ? total : kt;
  int32_t* out = tok + static_cast<int64_t>(row) * kt;
  for (uint32_t p = tid; p < static_cast<uint32_t>(kt); p += kXT) {
    int32_t v = -1;
    if (p < m) {  // the last block i < c with off[i] <= p holds output p
      int lo = 0, hi = c - 1;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (off[mid] <= p) lo = mid; else hi = mid - 1;
      }
      v = static_cast<int32_t>(static_cast<int64_t>(blk[lo]) * Bs + (p - off[lo]));
    }
    out[p] = v;
  }
  if (tid == 0 && tok_count) tok_count[row] = static_cast<int32_t>(m);
}

}  // namespace

hipError_t launch_index_k_compress(const tsd_compress_args& a, hipStream_t s) {
  if (a.B == 0 || a.max_blocks == 0) return hipSuccess;
  // token pages spanned by max_blocks blocks from any start, at most a row's
  int64_t pages = (static_cast<int64_t>(a.max_blocks) * a.block_size + kPage - 1) / kPage + 1;
  pages = pages < a.pt_stride ? pages : a.pt_stride;
  dim3 grid(static_cast<uint32_t>((pages + kCW - 1) / kCW), static_cast<uint32_t>(a.B));
  dim3 block(kCW * kWave);
  switch (a.block_size) {
    case 1: hipLaunchKernelGGL(index_k_compress_kernel<1>, grid, block, 0, s, a); break;
    case 2: hipLaunchKernelGGL(index_k_compress_kernel<2>, grid, block, 0, s, a); break;
    case 4: hipLaunchKernelGGL(index_k_compress_kernel<4>, grid, block, 0, s, a); break;
    case 8: hipLaunchKernelGGL(index_k_compress_kernel<8>, grid, block, 0, s, a); break;
    case 16: hipLaunchKernelGGL(index_k_compress_kernel<16>, grid, block, 0, s, a); break;
    case 32: hipLaunchKernelGGL(index_k_compress_kernel<32>, grid, block, 0, s, a); break;
    case 64: hipLaunchKernelGGL(index_k_compress_kernel<64>, grid, block, 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_expand_blocks(const int32_t* sel, const int32_t* count,
                                int rows, int kb, int Bs,
                                const int32_t* row_lens, int kt, int32_t* tok,
                                int32_t* tok_count, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  hipLaunchKernelGGL(expand_blocks_kernel, dim3(static_cast<uint32_t>(rows)),
                     dim3(kXT), 0, s, sel, count, kb, Bs, row_lens, kt, tok,
                     tok_count);
  return hipGetLastError();
}

}  // namespace tsd
