// C ABI of libpagedkv (declared in include/pagedkv.h): argument checks,
// kernel selection and launches. No allocation, no state, no host sync.
#include <math.h>

#include <map>
#include <mutex>
#include <tuple>

#include "launch.h"
#include "pagedkv.h"
#include "worklist.h"

using namespace pagedkv;

namespace {

constexpr int kMaxGroup = 16;
constexpr int kMaxGridYZ = 65535;
constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// Checks shared by every call: pool geometry and dtype.
// log2 of a supported block size (8 .. 256 tokens, a power of two), else -1
int block_shift(int block_size) {
  for (int sh = 3; sh <= 8; ++sh)
    if (block_size == (1 << sh)) return sh;
  return -1;
}

pa_status check_pool(const pa_dims* d) {
  if (!d) return PA_ERR_INVALID_ARG;
  if (block_shift(d->block_size) < 0) return PA_ERR_INVALID_ARG;
  if (d->num_kv_heads < 1 || d->head_dim < 1 || d->num_blocks < 1) return PA_ERR_INVALID_ARG;
  if (d->dtype != PA_F32 && d->dtype != PA_BF16) return PA_ERR_INVALID_ARG;
  if (d->head_dim != 64 && d->head_dim != 128) return PA_ERR_UNSUPPORTED;
  if (d->num_kv_heads > kMaxGridYZ) return PA_ERR_UNSUPPORTED;
  return PA_OK;
}

int elem_bytes(const pa_dims* d) { return d->dtype == PA_F32 ? 4 : 2; }

int pick_kernel(const pa_dims* d) {
  if (d->kernel != PA_KERNEL_AUTO) return d->kernel;
  return d->dtype == PA_BF16 ? PA_KERNEL_MFMA : PA_KERNEL_VALU;
}

// Balanced split: at most this many decode workgroups (4 waves each); the
// workspace holds two partial slots per wave. One workgroup per compute unit
// (256 on MI355X) streams faster than two: each wave's range is twice as
// long, so fewer pairs are cut, and the wave's own two-tile prefetch already
// keeps enough loads in flight.
constexpr int kMaxBalancedGrid = 256;
constexpr int kMinSegBlocks = 16;
// Chunked prefill: at most this many persistent workgroups.
constexpr int kMaxPrefillGrid = 1024;

// PA_PARTITION_AUTO: batches of at most kAutoFixedRows rows take the fixed
// split, larger ones the balanced split. A small batch leaves most of the
// balanced split's waves idle (each streams at least kMinSegBlocks tiles)
// and one wave merges each long row's many pieces, while the fixed split
// gives every (row, partition, KV head) its own workgroup: on the 32-layer
// 8B step it measured 20 us per layer at buckets 1-8 against 25-31 us
// balanced, and 12% slower at 32 rows.
constexpr int kAutoFixedRows = 8;
// The fixed split's partition length for B rows. Shorter partitions spread
// a row over more compute units (one streams a partition at about 30 GB/s);
// longer ones leave fewer partials for the merge, which one workgroup reads
// at that same rate. Measured on the 32-layer 8B step (bucket: real rows,
// us per layer for partitions of 192 / 256 / 320 / 384 / 512 tokens;
// two boxes agreed within 1%): bucket 1: 18.8 / 14.6 / 14.4 / 15.2 / 15.7;
// bucket 2: 10.8 / 11.9 / 12.5 / 13.6 / 13.9; bucket 4 (3 rows): 19.0 /
// 19.0 / 16.4 / 17.0 / 17.7; bucket 8 (5 rows): 18.0 / 17.5 / 16.6 / 16.3 /
// 17.6. A single row keeps 256 tokens, whose slots (rows x partitions x KV
// heads) fit the compute units at 8,192 tokens and 8 KV heads.
constexpr int auto_partition(int rows) {
  return rows <= 1 ? 256 : rows == 2 ? 192 : rows <= 4 ? 320 : 384;
}
constexpr int kAutoPartitionValu = 512;  // the vector-ALU kernel, any batch

struct Plan {
  int kernel;       // PA_KERNEL_VALU or PA_KERNEL_MFMA
  bool balanced;    // balanced split (MFMA, partition_tokens == 0)
  int partition;    // partition_tokens after resolving PA_PARTITION_AUTO
  int part_tokens;  // fixed split: tokens per partition (multiple of 16)
  int num_parts;    // fixed split: partitions per sequence at most
  size_t ws_bytes;  // 0 when nothing is ever merged
  size_t off_m, off_l, off_o;  // fp32 partials
  size_t off_cnt;              // balanced split: int32 piece counters [B, Hkv]
};

// balanced_only: the caller has only the balanced split (PA_PARTITION_AUTO
// then resolves to it).
pa_status plan_decode(const pa_dims* d, Plan* p, bool balanced_only = false) {
  pa_status st = check_pool(d);
  if (st != PA_OK) return st;
  if (d->num_seqs < 1 || d->num_q_heads < 1 || d->max_blocks_per_seq < 1)
    return PA_ERR_INVALID_ARG;
  if (d->num_q_heads % d->num_kv_heads != 0) return PA_ERR_INVALID_ARG;
  if (d->num_q_heads / d->num_kv_heads > kMaxGroup) return PA_ERR_UNSUPPORTED;
  if (d->num_seqs > kMaxSeqs || d->num_q_heads > kMaxGridYZ) return PA_ERR_UNSUPPORTED;
  if (d->max_blocks_per_seq > (1 << 26)) return PA_ERR_UNSUPPORTED;
  if (d->kernel != PA_KERNEL_AUTO && d->kernel != PA_KERNEL_VALU && d->kernel != PA_KERNEL_MFMA)
    return PA_ERR_INVALID_ARG;
  if (d->kernel == PA_KERNEL_MFMA && d->dtype != PA_BF16) return PA_ERR_UNSUPPORTED;
  p->kernel = pick_kernel(d);
  p->partition = d->partition_tokens;
  if (p->partition == PA_PARTITION_AUTO) {
    const bool fixed = p->kernel != PA_KERNEL_MFMA ||
                       (!balanced_only && d->block_size == kBlockTokens &&
                        d->num_seqs <= kAutoFixedRows);
    p->partition = !fixed ? 0
                   : p->kernel == PA_KERNEL_MFMA ? auto_partition(d->num_seqs)
                                                 : kAutoPartitionValu;
  }
  if (p->partition < 0 || p->partition % kBlockTokens != 0) return PA_ERR_INVALID_ARG;
  const int G = d->num_q_heads / d->num_kv_heads;
  const int max_tokens = d->max_blocks_per_seq * d->block_size;
  p->balanced = p->kernel == PA_KERNEL_MFMA && p->partition == 0;
  // blocks of other than 16 tokens: the balanced split only
  if (d->block_size != kBlockTokens && !p->balanced) return PA_ERR_UNSUPPORTED;
  if (p->balanced) {
    p->part_tokens = max_tokens;
    p->num_parts = 1;
    // counters, then one record per piece slot (two per wave): O, m, l
    const size_t slots = (size_t)2 * 4 * kMaxBalancedGrid;
    p->off_cnt = 0;
    p->off_o = align_up((size_t)d->num_seqs * d->num_kv_heads * sizeof(int));
    p->off_m = p->off_l = 0;
    p->ws_bytes = p->off_o + slots * (size_t)piece_floats(G, d->head_dim) * sizeof(float);
    return PA_OK;
  }
  const int part = (p->partition == 0 || p->partition >= max_tokens) ? max_tokens : p->partition;
  p->part_tokens = part;
  p->num_parts = (max_tokens + part - 1) / part;
  p->off_cnt = 0;
  if (p->num_parts == 1) {
    p->ws_bytes = p->off_m = p->off_l = p->off_o = 0;
    return PA_OK;
  }
  // partition counters per (sequence, KV head) (the matrix-core kernel
  // merges in place; the vector-ALU kernel leaves them to the reduce
  // kernel), then the partials: m, l, unnormalised output
  const size_t rows = (size_t)d->num_seqs * d->num_q_heads * p->num_parts;
  p->off_m = align_up((size_t)d->num_seqs * d->num_kv_heads * sizeof(int));
  p->off_l = p->off_m + align_up(rows * sizeof(float));
  p->off_o = p->off_l + align_up(rows * sizeof(float));
  p->ws_bytes = p->off_o + rows * (size_t)d->head_dim * sizeof(float);
  return PA_OK;
}

// Workgroups of `fn` (`threads` per workgroup, `smem` dynamic LDS bytes)
// the current device holds at once: CU count x occupancy. Cached per
// (device, kernel, LDS size rounded up to 1 KiB, threads); the only state
// the library keeps.
hipError_t resident_workgroups(const void* fn, size_t smem, int* out, int threads = 256) {
  static std::mutex mu;
  static std::map<std::tuple<int, const void*, size_t, int>, int> cache;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  smem = (smem + 1023) / 1024 * 1024;
  const auto key = std::make_tuple(dev, fn, smem, threads);
  std::lock_guard<std::mutex> lock(mu);
  auto it = cache.find(key);
  if (it != cache.end()) {
    *out = it->second;
    return hipSuccess;
  }
  int ncu = 0, per_cu = 0;
  e = hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, threads, smem);
  if (e != hipSuccess) return e;
  *out = cache[key] = (ncu > 0 ? ncu : 1) * (per_cu > 0 ? per_cu : 1);
  return hipSuccess;
}

// Compute units of the current device, cached per device.
hipError_t compute_units(int* out) {
  static std::mutex mu;
  static std::map<int, int> cache;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lock(mu);
  auto it = cache.find(dev);
  if (it != cache.end()) {
    *out = it->second;
    return hipSuccess;
  }
  int ncu = 0;
  e = hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  *out = cache[dev] = ncu > 0 ? ncu : 1;
  return hipSuccess;
}

// Dynamic LDS one workgroup may use on the current device, capped at the
// 160 KiB of a gfx950 compute unit and less 1 KiB for static LDS; cached
// per device.
hipError_t lds_per_workgroup(size_t* out) {
  static std::mutex mu;
  static std::map<int, size_t> cache;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lock(mu);
  auto it = cache.find(dev);
  if (it != cache.end()) {
    *out = it->second;
    return hipSuccess;
  }
  int bytes = 0;
  e = hipDeviceGetAttribute(&bytes, hipDeviceAttributeMaxSharedMemoryPerBlock, dev);
  if (e != hipSuccess) return e;
  size_t lim = bytes > 0 ? (size_t)bytes : 65536;
  if (lim > 160 * 1024) lim = 160 * 1024;
  *out = cache[dev] = lim - 1024;
  return hipSuccess;
}

// pa_decode, and pa_decode_append when k_new is non-null: the balanced split
// stores each row's new token inside the decode kernel; any other plan
// launches the KV append kernel first.
// With `contiguous`, k_pool / v_pool are unpaged caches (pa_decode_contiguous),
// block_tables is unused, and only the balanced split is taken.
pa_status decode_impl(const void* q, const void* k_new, const void* v_new,
                      const int32_t* slot_mapping, const void* k_pool, const void* v_pool,
                      const int32_t* block_tables, const int32_t* seq_lens, float scale,
                      void* out, const pa_dims* dims, void* workspace, size_t workspace_bytes,
                      void* stream, bool contiguous = false) {
  Plan plan;
  pa_status st = plan_decode(dims, &plan, contiguous);
  if (st != PA_OK) return st;
  if (contiguous && (!plan.balanced || dims->block_size != kBlockTokens))
    return PA_ERR_UNSUPPORTED;
  if (!q || !k_pool || !v_pool || (!block_tables && !contiguous) || !seq_lens || !out)
    return PA_ERR_INVALID_ARG;
  if (!isfinite(scale)) return PA_ERR_INVALID_ARG;
  if (plan.ws_bytes > 0 && (!workspace || workspace_bytes < plan.ws_bytes))
    return PA_ERR_INVALID_ARG;

  DecodeArgs a;
  a.q = q;
  a.k_pool = k_pool;
  a.v_pool = v_pool;
  a.block_tables = block_tables;
  a.seq_lens = seq_lens;
  a.out = out;
  char* ws = (char*)workspace;
  a.ws_m = plan.ws_bytes && !plan.balanced ? (float*)(ws + plan.off_m) : nullptr;
  a.ws_l = plan.ws_bytes && !plan.balanced ? (float*)(ws + plan.off_l) : nullptr;
  a.ws_o = plan.ws_bytes ? (float*)(ws + plan.off_o) : nullptr;
  a.ws_cnt = plan.ws_bytes ? (int*)(ws + plan.off_cnt) : nullptr;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.num_seqs = dims->num_seqs;
  a.num_q_heads = dims->num_q_heads;
  a.num_kv_heads = dims->num_kv_heads;
  a.group = dims->num_q_heads / dims->num_kv_heads;
  a.max_blocks = dims->max_blocks_per_seq;
  a.part_tokens = plan.part_tokens;
  a.num_parts = plan.num_parts;
  a.split_waves = 0;
  a.min_seg_blocks = 0;
  a.stage_slots = 0;
  a.slot_grid = 0;
  a.block_shift = block_shift(dims->block_size);
  a.k_new = nullptr;
  a.v_new = nullptr;
  a.slot_mapping = nullptr;

  hipStream_t s = (hipStream_t)stream;
  hipError_t e = hipSuccess;
  if (k_new != nullptr) {
    if (plan.balanced) {
      a.k_new = k_new;
      a.v_new = v_new;
      a.slot_mapping = slot_mapping;
    } else {
      e = launch_write_kv(k_new, v_new, slot_mapping, dims->num_seqs, (void*)k_pool,
                          (void*)v_pool, dims->num_kv_heads, dims->head_dim,
                          block_shift(dims->block_size), elem_bytes(dims), s);
      if (e != hipSuccess) return PA_ERR_LAUNCH;
    }
  }
  if (plan.balanced) {
    size_t lds = 0;
    e = lds_per_workgroup(&lds);
    if (e != hipSuccess) return PA_ERR_LAUNCH;
    a.stage_slots = balanced_stage_slots(dims->num_seqs, a.group, dims->head_dim, lds);
    if (decode_mfma_smem(dims->num_seqs, a.group, dims->head_dim, true, 0) > lds)
      return PA_ERR_UNSUPPORTED;  // the work list and parked pieces alone do not fit
  }
  const void* fn = plan.kernel == PA_KERNEL_MFMA
                       ? decode_mfma_fn(dims->head_dim, plan.balanced, a.block_shift, contiguous)
                       : decode_valu_fn(dims->dtype, dims->head_dim, a.group);
  const size_t smem = plan.kernel == PA_KERNEL_MFMA
                          ? decode_mfma_smem(dims->num_seqs, a.group, dims->head_dim,
                                             plan.balanced, a.stage_slots)
                          : (size_t)(dims->num_seqs + 1) * sizeof(int);
  int resident = 0;
  e = resident_workgroups(fn, smem, &resident);
  if (e != hipSuccess) return PA_ERR_LAUNCH;
  if (plan.balanced) {
    const int grid = resident < kMaxBalancedGrid ? resident : kMaxBalancedGrid;
    a.split_waves = 4 * grid;
    a.min_seg_blocks = kMinSegBlocks;
    e = launch_decode_mfma(a, dims->head_dim, true, grid, s, contiguous);
    return e == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
  }
  // never more workgroups than items can exist
  const long long max_items = (long long)dims->num_seqs * dims->num_kv_heads * plan.num_parts;
  int grid = (int)(max_items < resident ? max_items : resident);
  if (plan.kernel == PA_KERNEL_MFMA) {
    // When every (row, partition, KV head) slot fits on a compute unit of
    // its own, each slot gets a workgroup and no work list is built: the
    // row length, queries and first table entries load together. A
    // compute unit streams at a fixed rate, so with more slots than compute
    // units the work list's packing of the real items onto distinct
    // compute units is worth its cost.
    int ncu = 0;
    e = compute_units(&ncu);
    if (e != hipSuccess) return PA_ERR_LAUNCH;
    if (max_items <= ncu && max_items <= resident) {
      a.slot_grid = 1;
      grid = (int)max_items;
    }
    e = launch_decode_mfma(a, dims->head_dim, false, grid, s);
  }
  else
    e = launch_decode_valu(a, dims->dtype, dims->head_dim, grid, s);
  if (e != hipSuccess) return PA_ERR_LAUNCH;
  if (plan.num_parts > 1 && plan.kernel != PA_KERNEL_MFMA) {
    e = launch_decode_reduce(a, dims->dtype, dims->head_dim, s);
    if (e != hipSuccess) return PA_ERR_LAUNCH;
  }
  return PA_OK;
}

// ---- allocation-free decode -----------------------------------------------
//
// pa_decode_noalloc's workspace: a device array of the library's own, one
// copy per GPU, held until the process ends. In host code `scratch` names a
// host-side stand-in, never the device memory: the device address comes
// from hipGetSymbolAddress, once per device with that device current, and
// only that address is passed to kernels.
constexpr size_t kScratchBytes = PA_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

hipError_t scratch_address(void** out) {
  static std::mutex mu;
  static std::map<int, void*> cache;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lock(mu);
  auto it = cache.find(dev);
  if (it != cache.end()) {
    *out = it->second;
    return hipSuccess;
  }
  void* ptr = nullptr;
  e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
  if (e != hipSuccess) return e;
  if (ptr == nullptr) return hipErrorInvalidSymbol;
  *out = cache[dev] = ptr;
  return hipSuccess;
}

// Latent decode: one workgroup per compute unit, at most this many; a
// workgroup's range holds at least kLatentMinTiles 32-token tiles.
constexpr int kMaxLatentGrid = 256;
constexpr int kLatentMinTiles = 8;

struct LatentPlan {
  size_t off_cnt, off_rec, ws_bytes;
};

pa_status plan_latent(const pa_latent_dims* d, LatentPlan* p) {
  if (!d) return PA_ERR_INVALID_ARG;
  if (d->num_seqs < 1 || d->num_heads < 1 || d->latent_dim < 1 || d->value_dim < 1 ||
      d->block_size < 1 || d->max_blocks_per_seq < 1 || d->num_blocks < 1)
    return PA_ERR_INVALID_ARG;
  if (d->dtype != PA_F32 && d->dtype != PA_BF16) return PA_ERR_INVALID_ARG;
  if (d->value_dim > d->latent_dim) return PA_ERR_INVALID_ARG;
  if (d->dtype != PA_BF16 || d->num_heads != kLatentHeads || d->latent_dim != kLatentDim ||
      d->value_dim != kLatentValueDim || d->block_size != kLatentBlockTokens)
    return PA_ERR_UNSUPPORTED;
  if (d->num_seqs > kMaxSeqs || d->max_blocks_per_seq > (1 << 20)) return PA_ERR_UNSUPPORTED;
  const size_t B = (size_t)d->num_seqs;
  p->off_cnt = 0;
  p->off_rec = align_up(2 * B * sizeof(int));
  p->ws_bytes = p->off_rec + (size_t)2 * kMaxLatentGrid * kLatentRecordBytes;
  return PA_OK;
}

}  // namespace

extern "C" {

size_t pa_latent_workspace_bytes(const pa_latent_dims* dims) {
  LatentPlan p;
  if (plan_latent(dims, &p) != PA_OK) return 0;
  return p.ws_bytes;
}

pa_status pa_latent_decode(const void* q, const void* kv_pool, const int32_t* block_tables,
                           const int32_t* seq_lens, float scale, void* out,
                           const pa_latent_dims* dims, void* workspace, size_t workspace_bytes,
                           void* stream) {
  LatentPlan plan;
  pa_status st = plan_latent(dims, &plan);
  if (st != PA_OK) return st;
  if (!q || !kv_pool || !block_tables || !seq_lens || !out) return PA_ERR_INVALID_ARG;
  if (!isfinite(scale)) return PA_ERR_INVALID_ARG;
  if (!workspace || workspace_bytes < plan.ws_bytes) return PA_ERR_INVALID_ARG;
  size_t lds = 0;
  hipError_t e = lds_per_workgroup(&lds);
  if (e != hipSuccess) return PA_ERR_LAUNCH;
  const size_t smem = latent_decode_smem(dims->num_seqs);
  if (smem > lds) return PA_ERR_UNSUPPORTED;
  int resident = 0;
  e = resident_workgroups(latent_decode_fn(), smem, &resident);
  if (e != hipSuccess) return PA_ERR_LAUNCH;
  char* ws = (char*)workspace;
  LatentArgs a;
  a.q = q;
  a.kv_pool = kv_pool;
  a.block_tables = block_tables;
  a.seq_lens = seq_lens;
  a.out = out;
  a.ws_rec = (float*)(ws + plan.off_rec);
  a.ws_cnt = (int*)(ws + plan.off_cnt);
  a.scale_log2 = scale * 1.4426950408889634f;
  a.num_seqs = dims->num_seqs;
  a.max_blocks = dims->max_blocks_per_seq;
  a.grid = resident < kMaxLatentGrid ? resident : kMaxLatentGrid;
  a.min_tiles = kLatentMinTiles;
  e = launch_latent_decode(a, (hipStream_t)stream);
  return e == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

pa_status pa_latent_write(const void* kv_new, const int32_t* slot_mapping, int32_t num_tokens,
                          void* kv_pool, const pa_latent_dims* dims, void* stream) {
  LatentPlan plan;
  pa_status st = plan_latent(dims, &plan);
  if (st != PA_OK) return st;
  if (num_tokens < 0) return PA_ERR_INVALID_ARG;
  if (num_tokens == 0) return PA_OK;
  if (!kv_new || !slot_mapping || !kv_pool) return PA_ERR_INVALID_ARG;
  hipError_t e = launch_latent_write(kv_new, slot_mapping, num_tokens, kv_pool,
                                     (hipStream_t)stream);
  return e == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}


size_t pa_decode_workspace_bytes(const pa_dims* dims) {
  Plan p;
  if (plan_decode(dims, &p) != PA_OK) return 0;
  return p.ws_bytes;
}

pa_status pa_decode(const void* q, const void* k_pool, const void* v_pool,
                    const int32_t* block_tables, const int32_t* seq_lens, float scale,
                    void* out, const pa_dims* dims, void* workspace, size_t workspace_bytes,
                    void* stream) {
  return decode_impl(q, nullptr, nullptr, nullptr, k_pool, v_pool, block_tables, seq_lens, scale,
                     out, dims, workspace, workspace_bytes, stream);
}

pa_status pa_decode_contiguous(const void* q, const void* k_cache, const void* v_cache,
                               const int32_t* seq_lens, float scale, void* out,
                               const pa_dims* dims, void* workspace, size_t workspace_bytes,
                               void* stream) {
  return decode_impl(q, nullptr, nullptr, nullptr, k_cache, v_cache, nullptr, seq_lens, scale,
                     out, dims, workspace, workspace_bytes, stream, true);
}

pa_status pa_decode_noalloc(const void* q, const void* k_pool, const void* v_pool,
                            const int32_t* block_tables, const int32_t* seq_lens, float scale,
                            void* out, const pa_dims* dims, void* stream) {
  Plan plan;
  pa_status st = plan_decode(dims, &plan);
  if (st != PA_OK) return st;
  if (plan.ws_bytes > kScratchBytes) return PA_ERR_UNSUPPORTED;
  if (!q || !k_pool || !v_pool || !block_tables || !seq_lens || !out) return PA_ERR_INVALID_ARG;
  if (!isfinite(scale)) return PA_ERR_INVALID_ARG;
  void* ws = nullptr;
  if (scratch_address(&ws) != hipSuccess) return PA_ERR_LAUNCH;
  if (plan.ws_bytes > 0) {
    // the piece or partition counters must start at zero; the previous call
    // on this GPU left them so unless it failed or had other dims, and the
    // fill makes it certain
    const size_t end = plan.balanced ? plan.off_o : plan.off_m;
    const hipError_t e =
        launch_zero_fill((char*)ws + plan.off_cnt, end - plan.off_cnt, (hipStream_t)stream);
    if (e != hipSuccess) return PA_ERR_LAUNCH;
  }
  return decode_impl(q, nullptr, nullptr, nullptr, k_pool, v_pool, block_tables, seq_lens, scale,
                     out, dims, ws, kScratchBytes, stream);
}

pa_status pa_decode_append(const void* q, const void* k_new, const void* v_new,
                           const int32_t* slot_mapping, void* k_pool, void* v_pool,
                           const int32_t* block_tables, const int32_t* seq_lens, float scale,
                           void* out, const pa_dims* dims, void* workspace,
                           size_t workspace_bytes, void* stream) {
  if (!k_new || !v_new || !slot_mapping) return PA_ERR_INVALID_ARG;
  return decode_impl(q, k_new, v_new, slot_mapping, k_pool, v_pool, block_tables, seq_lens,
                     scale, out, dims, workspace, workspace_bytes, stream);
}

pa_status pa_prefill(const void* q, const void* k_pool, const void* v_pool,
                     const int32_t* block_tables, const int32_t* seq_lens,
                     const int32_t* query_start, int32_t num_query_tokens, float scale,
                     void* out, const pa_dims* dims, void* stream) {
  pa_status st = check_pool(dims);
  if (st != PA_OK) return st;
  if (dims->num_seqs < 1 || dims->num_q_heads < 1 || dims->max_blocks_per_seq < 1)
    return PA_ERR_INVALID_ARG;
  if (dims->num_q_heads % dims->num_kv_heads != 0) return PA_ERR_INVALID_ARG;
  if (num_query_tokens < 0) return PA_ERR_INVALID_ARG;
  if (dims->dtype != PA_BF16 || dims->block_size < kBlockTokens) return PA_ERR_UNSUPPORTED;
  if (dims->num_seqs > kMaxSeqs || dims->max_blocks_per_seq > (1 << 26))
    return PA_ERR_UNSUPPORTED;
  if (num_query_tokens == 0) return PA_OK;
  if (!q || !k_pool || !v_pool || !block_tables || !seq_lens || !query_start || !out)
    return PA_ERR_INVALID_ARG;
  // positive: the kernel takes each column's max before scaling
  if (!isfinite(scale) || !(scale > 0.f)) return PA_ERR_INVALID_ARG;

  PrefillArgs a;
  a.q = q;
  a.k_pool = k_pool;
  a.v_pool = v_pool;
  a.block_tables = block_tables;
  a.seq_lens = seq_lens;
  a.query_start = query_start;
  a.out = out;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.num_seqs = dims->num_seqs;
  a.num_q_heads = dims->num_q_heads;
  a.num_kv_heads = dims->num_kv_heads;
  a.group = dims->num_q_heads / dims->num_kv_heads;
  a.max_blocks = dims->max_blocks_per_seq;
  a.block_shift = block_shift(dims->block_size);
  size_t lds = 0;
  hipError_t e = lds_per_workgroup(&lds);
  if (e != hipSuccess) return PA_ERR_LAUNCH;
  const size_t smem = prefill_mfma_smem(dims->num_seqs, dims->head_dim);
  if (smem > lds) return PA_ERR_UNSUPPORTED;
  int resident = 0;
  e = resident_workgroups(prefill_mfma_fn(dims->head_dim), smem, &resident, kPrefillThreads);
  if (e != hipSuccess) return PA_ERR_LAUNCH;
  const int grid = resident < kMaxPrefillGrid ? resident : kMaxPrefillGrid;
  e = launch_prefill_mfma(a, dims->head_dim, grid, (hipStream_t)stream);
  return e == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

pa_status pa_write_kv(const void* k_new, const void* v_new, const int32_t* slot_mapping,
                      int32_t num_tokens, void* k_pool, void* v_pool, const pa_dims* dims,
                      void* stream) {
  pa_status st = check_pool(dims);
  if (st != PA_OK) return st;
  if (num_tokens < 0) return PA_ERR_INVALID_ARG;
  if (num_tokens == 0) return PA_OK;
  if (!k_new || !v_new || !slot_mapping || !k_pool || !v_pool) return PA_ERR_INVALID_ARG;
  hipError_t e = launch_write_kv(k_new, v_new, slot_mapping, num_tokens, k_pool, v_pool,
                                 dims->num_kv_heads, dims->head_dim,
                                 block_shift(dims->block_size), elem_bytes(dims),
                                 (hipStream_t)stream);
  return e == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

pa_status pa_copy_blocks(void* k_pool, void* v_pool, const int32_t* block_mapping,
                         int32_t num_pairs, const pa_dims* dims, void* stream) {
  pa_status st = check_pool(dims);
  if (st != PA_OK) return st;
  if (num_pairs < 0) return PA_ERR_INVALID_ARG;
  if (num_pairs == 0) return PA_OK;
  if (!k_pool || !v_pool || !block_mapping) return PA_ERR_INVALID_ARG;
  const size_t block_bytes =
      (size_t)dims->num_kv_heads * dims->block_size * dims->head_dim * elem_bytes(dims);
  hipError_t e = launch_copy_blocks(k_pool, v_pool, block_mapping, num_pairs, block_bytes,
                                    (hipStream_t)stream);
  return e == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

const char* pa_status_string(pa_status status) {
  switch (status) {
    case PA_OK: return "ok";
    case PA_ERR_INVALID_ARG: return "invalid argument";
    case PA_ERR_UNSUPPORTED: return "unsupported configuration";
    case PA_ERR_LAUNCH: return "kernel launch failed";
  }
  return "unknown status";
}

const char* pa_version(void) { return "pagedkv 0.1 gfx950"; }

}  // extern "C"
