// Host entry points of the C ABI declared in include/mla.h: argument
// validation (before any launch), kernel selection and launch on the
// caller's stream.  The library allocates nothing and keeps no state.
#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <vector>

#include "mla.h"
#include "mla_kernels.h"
#include "gate_kernels.h"

namespace {

constexpr int kDL = 512, kDR = 64, kDH = 128, kBlock = 64;

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int elem_size(int32_t dt) {
  switch (dt) {
    case MLA_F32: return 4;
    case MLA_BF16: return 2;
    case MLA_FP8_E4M3: return 1;
    default: return 0;
  }
}

// MLA_CHECK=1 in the environment at the call: mla_decode validates the
// device-side paging data before launching (read back on the stream).
bool check_mode() {
  const char* e = getenv("MLA_CHECK");
  return e && e[0] == '1' && e[1] == 0;
}

// Every length in [0, max_blocks_per_seq * block_size] and every block id a
// sequence uses (its first ceil(len / block_size) table entries) in
// [0, num_blocks); MLA_ERR_DEVICE if the read-back fails.
int check_paging(int32_t batch, const mla_paged_kv* kv, hipStream_t s) {
  std::vector<int32_t> lens((size_t)batch), table((size_t)batch * kv->max_blocks_per_seq);
  if (hipMemcpyAsync(lens.data(), kv->seq_lens, lens.size() * 4, hipMemcpyDeviceToHost, s) != hipSuccess ||
      hipMemcpyAsync(table.data(), kv->block_table, table.size() * 4, hipMemcpyDeviceToHost, s) != hipSuccess ||
      hipStreamSynchronize(s) != hipSuccess)
    return MLA_ERR_DEVICE;
  for (int32_t b = 0; b < batch; ++b) {
    const int64_t len = lens[b];
    if (len < 0 || len > (int64_t)kv->max_blocks_per_seq * kv->block_size) return MLA_ERR_SHAPE;
    const int64_t pages = (len + kv->block_size - 1) / kv->block_size;
    for (int64_t p = 0; p < pages; ++p) {
      const int32_t blk = table[(size_t)b * kv->max_blocks_per_seq + p];
      if (blk < 0 || blk >= kv->num_blocks) return MLA_ERR_SHAPE;
    }
  }
  return MLA_OK;
}

int check_dims(const mla_dims* d) {
  if (!d) return MLA_ERR_NULL;
  if (d->batch < 0 || d->heads < 1 || d->heads > 1024 || d->q_per_seq < 1 || d->q_per_seq > MLA_MAX_Q_PER_SEQ)
    return MLA_ERR_SHAPE;
  if (d->d_latent != kDL || d->d_rope != kDR || d->d_head != kDH) return MLA_ERR_SHAPE;
  if (!isfinite(d->softmax_scale)) return MLA_ERR_SHAPE;
  // row counts must fit 32-bit index arithmetic in the kernels
  if ((int64_t)d->batch * d->q_per_seq * d->heads > (1 << 24)) return MLA_ERR_SHAPE;
  return MLA_OK;
}

// MLA_DECODE_ROWS=64 or 32 in the environment at the call fixes the bf16
// decode's query rows per workgroup (otherwise chosen from the launch size).
int forced_decode_rows() {
  const char* e = getenv("MLA_DECODE_ROWS");
  if (!e) return 0;
  if (!strcmp(e, "64")) return 64;
  if (!strcmp(e, "32")) return 32;
  return 0;
}

// Compute units of the current device (0 if unknown; cached per device).
int device_cus() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  if (!cached[dev]) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    cached[dev] = cus;
  }
  return cached[dev];
}

// Launch through hipLaunchKernel so the status returned is this launch's own
// (hipGetLastError would also report errors left by unrelated earlier calls).
// With MLA_VERBOSE set in the environment a refused launch prints the HIP error.
template <typename Args>
int launch(const char* name, const void* kernel, dim3 grid, dim3 block, const Args& a, hipStream_t s) {
  void* argv[] = {(void*)&a};
  const hipError_t e = hipLaunchKernel(kernel, grid, block, argv, 0, s);
  if (e == hipSuccess) return MLA_OK;
  if (getenv("MLA_VERBOSE"))
    fprintf(stderr, "mla: launch of %s (grid %u,%u,%u block %u) failed: %s\n", name, grid.x, grid.y, grid.z,
            block.x, hipGetErrorString(e));
  return MLA_ERR_LAUNCH;
}

}  // namespace

extern "C" {

const char* mla_status_str(int status) {
  switch (status) {
    case MLA_OK: return "MLA_OK";
    case MLA_ERR_NULL: return "MLA_ERR_NULL: a required pointer is NULL";
    case MLA_ERR_SHAPE: return "MLA_ERR_SHAPE: a size is out of range or unsupported";
    case MLA_ERR_DTYPE: return "MLA_ERR_DTYPE: unsupported dtype or dtype combination";
    case MLA_ERR_ALIGN: return "MLA_ERR_ALIGN: a pointer or stride is not 16-byte aligned";
    case MLA_ERR_SPLITS: return "MLA_ERR_SPLITS: num_splits out of range";
    case MLA_ERR_LAUNCH: return "MLA_ERR_LAUNCH: the HIP runtime refused the launch";
    case MLA_ERR_DEVICE: return "MLA_ERR_DEVICE: no usable device";
    case MLA_ERR_SCRATCH: return "MLA_ERR_SCRATCH: the call needs more than the library's static scratch holds";
    default: return "MLA_ERR_UNKNOWN";
  }
}

int mla_abi_version(void) { return MLA_ABI_VERSION; }

// The build passes the hash of the sources; the prefix lets a build check
// find it in the library file without loading it.
#ifndef MLA_SOURCE_HASH
#define MLA_SOURCE_HASH "0000000000000000"
#endif
static const char kSourceHash[] = "mla-source-hash:" MLA_SOURCE_HASH;
static_assert(sizeof(kSourceHash) == 16 + 16 + 1, "the source hash is 16 hex digits");

const char* mla_source_hash(void) { return kSourceHash + 16; }

int mla_absorb_q(const mla_dims* dims, const void* q_nope, const void* w_uk, int32_t in_dtype,
                 void* q_lat, int32_t q_lat_dtype, void* stream) {
  int st = check_dims(dims);
  if (st) return st;
  if (!q_nope || !w_uk || !q_lat) return MLA_ERR_NULL;
  if ((in_dtype != MLA_F32 && in_dtype != MLA_BF16) || (q_lat_dtype != MLA_F32 && q_lat_dtype != MLA_BF16))
    return MLA_ERR_DTYPE;
  if (!aligned16(q_nope) || !aligned16(w_uk) || !aligned16(q_lat)) return MLA_ERR_ALIGN;
  const int rows = dims->batch * dims->q_per_seq;
  if (rows == 0) return MLA_OK;
  mla::AbsorbArgs a{q_nope, w_uk, q_lat, rows, dims->heads};
  hipStream_t s = (hipStream_t)stream;
  if (in_dtype == MLA_BF16) {
    dim3 grid(dims->heads * 4);  // (head, quarter of d_latent)
    if (q_lat_dtype == MLA_BF16)
      st = launch("mla::absorb_q_mfma<true>", (const void*)mla::absorb_q_mfma<true>, grid, dim3(256), a, s);
    else
      st = launch("mla::absorb_q_mfma<false>", (const void*)mla::absorb_q_mfma<false>, grid, dim3(256), a, s);
  } else {
    dim3 grid(dims->heads * (kDL / 64));  // (head, block of 64 latent columns)
    if (rows > 65535) return MLA_ERR_SHAPE;
    if (q_lat_dtype == MLA_BF16)
      st = launch("mla::absorb_q_f32<true>", (const void*)mla::absorb_q_f32<true>, grid, dim3(256), a, s);
    else
      st = launch("mla::absorb_q_f32<false>", (const void*)mla::absorb_q_f32<false>, grid, dim3(256), a, s);
  }
  return st;
}

int mla_decode(const mla_dims* dims, const void* q_lat, const void* q_rope, int32_t q_dtype,
               const mla_paged_kv* kv, int32_t num_splits, void* o, int32_t o_dtype, float* lse, void* stream) {
  int st = check_dims(dims);
  if (st) return st;
  if (!kv || !q_lat || !q_rope || !o || !lse) return MLA_ERR_NULL;
  if (!kv->latent || !kv->rope || !kv->block_table || !kv->seq_lens) return MLA_ERR_NULL;
  if (num_splits < 1 || num_splits > MLA_MAX_SPLITS) return MLA_ERR_SPLITS;
  if (kv->block_size != kBlock || kv->num_blocks < 1 || kv->max_blocks_per_seq < 1) return MLA_ERR_SHAPE;
  const int32_t ld = kv->latent_dtype, rd = kv->rope_dtype;
  int fmt;  // 0 = f32, 1 = bf16, 2 = fp8
  if (q_dtype == MLA_F32 && ld == MLA_F32 && rd == MLA_F32) fmt = 0;
  else if (q_dtype == MLA_BF16 && ld == MLA_BF16 && rd == MLA_BF16) fmt = 1;
  else if (q_dtype == MLA_BF16 && ld == MLA_FP8_E4M3 && rd == MLA_BF16) fmt = 2;
  else return MLA_ERR_DTYPE;
  if (fmt == 2 && !kv->scale) return MLA_ERR_NULL;
  if (fmt != 2 && kv->scale) return MLA_ERR_DTYPE;
  // fp16 chunk partials: split bf16 / fp8 decodes only
  if (o_dtype != MLA_F32 && !(o_dtype == MLA_F16 && num_splits > 1 && fmt != 0)) return MLA_ERR_DTYPE;
  if (kv->latent_row_stride < kDL || kv->rope_row_stride < kDR || kv->latent_block_stride < 0 ||
      kv->rope_block_stride < 0 || (fmt == 2 && kv->scale_block_stride < kBlock))
    return MLA_ERR_SHAPE;
  const int64_t les = elem_size(ld), res = elem_size(rd);
  const int64_t lat_rs = kv->latent_row_stride * les, lat_bs = kv->latent_block_stride * les;
  const int64_t rope_rs = kv->rope_row_stride * res, rope_bs = kv->rope_block_stride * res;
  if (!aligned16(q_lat) || !aligned16(q_rope) || !aligned16(o) || !aligned16(kv->latent) ||
      !aligned16(kv->rope) || (lat_rs & 15) || (lat_bs & 15) || (rope_rs & 15) || (rope_bs & 15) ||
      (fmt == 2 && (((uintptr_t)kv->scale & 15) || (kv->scale_block_stride & 3))))
    return MLA_ERR_ALIGN;
  const int rows = dims->q_per_seq * dims->heads;
  if (dims->batch == 0) return MLA_OK;
  const int64_t units = (int64_t)dims->batch * num_splits;
  if (units > (1 << 24)) return MLA_ERR_SHAPE;
  if (check_mode()) {
    st = check_paging(dims->batch, kv, (hipStream_t)stream);
    if (st) return st;
  }

  mla::DecodeArgs a;
  a.q_lat = (const uint16_t*)q_lat;
  a.q_rope = (const uint16_t*)q_rope;
  a.latent = (const uint8_t*)kv->latent;
  a.rope = (const uint8_t*)kv->rope;
  a.kv_scale_bytes = (const uint8_t*)kv->scale;
  a.lat_bs = lat_bs;
  a.lat_rs = lat_rs;
  a.rope_bs = rope_bs;
  a.rope_rs = rope_rs;
  a.scale_bs = (int64_t)kv->scale_block_stride * 4;
  a.block_table = kv->block_table;
  a.seq_lens = kv->seq_lens;
  a.o = o;
  a.lse = lse;
  a.o_f16 = o_dtype == MLA_F16;
  a.batch = dims->batch;
  a.sq = dims->q_per_seq;
  a.heads = dims->heads;
  a.rows = rows;
  // bf16: 32-row workgroups when 64-row ones would leave compute units idle
  // (few (sequence, chunk) units: a long context split into few chunks)
  int rows_per_wg = mla::kDecodeRowsPerWg;
  if (fmt == 1) {
    const int forced = forced_decode_rows();
    if (forced) rows_per_wg = forced;
    else if (rows > 32 && units * ((rows + 63) / 64) < device_cus()) rows_per_wg = 32;
  }
  a.row_blocks = (rows + rows_per_wg - 1) / rows_per_wg;
  a.num_splits = num_splits;
  a.units = (int)units;
  a.max_blocks = kv->max_blocks_per_seq;
  a.softmax_scale = dims->softmax_scale;
  a.scale_log2 = dims->softmax_scale * 1.4426950408889634f;
  hipStream_t s = (hipStream_t)stream;
  if (fmt == 1 || fmt == 2) {
    // matrix-core kernels: 8 waves per (sequence, chunk, row block), a
    // multiple of the 8 XCDs (see the kernels' placement)
    const int64_t grid = (units * a.row_blocks + 7) / 8 * 8;
    if (grid > 0x7fffffff) return MLA_ERR_SHAPE;
    if (fmt == 1 && rows_per_wg == 32)
      st = launch("mla::decode_mfma_bf16<32>", (const void*)mla::decode_mfma_bf16<32>, dim3((unsigned)grid), dim3(512),
                  a, s);
    else if (fmt == 1)
      st = launch("mla::decode_mfma_bf16<64>", (const void*)mla::decode_mfma_bf16<64>, dim3((unsigned)grid), dim3(512),
                  a, s);
    else
      st = launch("mla::decode_mfma_fp8", (const void*)mla::decode_mfma_fp8, dim3((unsigned)grid), dim3(512), a, s);
  } else {
    const int64_t grid = (units * rows + 7) / 8 * 8;  // a multiple of the 8 XCDs (see the kernel's placement)
    if (grid > 0x7fffffff) return MLA_ERR_SHAPE;
    st = launch("mla::decode_f32", (const void*)mla::decode_f32, dim3((unsigned)grid), dim3(512), a, s);
  }
  return st;
}

int mla_split_combine(const mla_dims* dims, int32_t num_splits, const void* o_part, int32_t part_dtype,
                      const float* lse_part, float* o_lat, float* lse, void* stream) {
  int st = check_dims(dims);
  if (st) return st;
  if (!o_part || !lse_part || !o_lat) return MLA_ERR_NULL;
  if (part_dtype != MLA_F32 && part_dtype != MLA_F16) return MLA_ERR_DTYPE;
  if (num_splits < 1 || num_splits > MLA_MAX_SPLITS) return MLA_ERR_SPLITS;
  if (!aligned16(o_part) || !aligned16(o_lat)) return MLA_ERR_ALIGN;
  const int rows = dims->q_per_seq * dims->heads;
  const int64_t total = (int64_t)dims->batch * rows;
  if (total == 0) return MLA_OK;
  mla::CombineArgs a{o_part, lse_part, o_lat, lse, dims->batch, num_splits, rows};
  // few chunks: a wave per row, four rows per workgroup; many: a workgroup per row
  const bool solo = num_splits <= mla::kCombineSoloMaxSplits;
  const bool f16 = part_dtype == MLA_F16;
  const void* k = solo ? (f16 ? (const void*)mla::split_combine<_Float16, true> : (const void*)mla::split_combine<float, true>)
                       : (f16 ? (const void*)mla::split_combine<_Float16, false> : (const void*)mla::split_combine<float, false>);
  const int64_t grid = solo ? (total + 3) / 4 : total;
  st = launch("mla::split_combine", k, dim3((unsigned)grid), dim3(256), a, (hipStream_t)stream);
  return st;
}

int mla_out_uv(const mla_dims* dims, const float* o_lat, const void* w_uv, int32_t w_dtype, void* out,
               int32_t out_dtype, void* stream) {
  int st = check_dims(dims);
  if (st) return st;
  if (!o_lat || !w_uv || !out) return MLA_ERR_NULL;
  if (w_dtype != MLA_F32 && w_dtype != MLA_BF16) return MLA_ERR_DTYPE;
  if (out_dtype != MLA_F32 && out_dtype != MLA_BF16) return MLA_ERR_DTYPE;
  if (!aligned16(o_lat) || !aligned16(w_uv) || !aligned16(out)) return MLA_ERR_ALIGN;
  const int rows = dims->batch * dims->q_per_seq;
  if (rows == 0) return MLA_OK;
  mla::OutUvArgs a{o_lat, w_uv, out, rows, dims->heads, nullptr, nullptr, nullptr, 1, dims->q_per_seq,
                   out_dtype == MLA_BF16, 0};
  hipStream_t s = (hipStream_t)stream;
  if (w_dtype == MLA_BF16) {
    st = launch("mla::out_uv_mfma", (const void*)mla::out_uv_mfma, dim3((dims->heads + 7) / 8 * 16),
                dim3(256), a, s);
  } else {
    if (rows > 65535) return MLA_ERR_SHAPE;
    st = launch("mla::out_uv_f32", (const void*)mla::out_uv_f32<false>, dim3(dims->heads * (kDH / 16)), dim3(256), a,
                s);
  }
  return st;
}

int mla_combine_out_uv(const mla_dims* dims, int32_t num_splits, const void* o_part, int32_t part_dtype,
                       const float* lse_part, const void* w_uv, int32_t w_dtype, void* out, int32_t out_dtype,
                       float* lse, void* stream) {
  int st = check_dims(dims);
  if (st) return st;
  if (!o_part || !lse_part || !w_uv || !out) return MLA_ERR_NULL;
  if (part_dtype != MLA_F32 && part_dtype != MLA_F16) return MLA_ERR_DTYPE;
  if (num_splits < 1 || num_splits > MLA_MAX_SPLITS) return MLA_ERR_SPLITS;
  if (w_dtype != MLA_F32 && w_dtype != MLA_BF16) return MLA_ERR_DTYPE;
  if (out_dtype != MLA_F32 && out_dtype != MLA_BF16) return MLA_ERR_DTYPE;
  if (!aligned16(o_part) || !aligned16(w_uv) || !aligned16(out)) return MLA_ERR_ALIGN;
  const int rows = dims->batch * dims->q_per_seq;
  if (rows == 0) return MLA_OK;
  mla::OutUvArgs a{nullptr, w_uv, out, rows, dims->heads, o_part, lse_part, lse, num_splits, dims->q_per_seq,
                   out_dtype == MLA_BF16, part_dtype == MLA_F16};
  hipStream_t s = (hipStream_t)stream;
  if (w_dtype == MLA_BF16 && num_splits > 8 && rows <= mla::kMergeFewRows) {
    // few query rows, many chunks: the chunks of a row spread over a workgroup
    const int64_t grid = (int64_t)dims->heads * 2;
    const void* k = part_dtype == MLA_F16 ? (const void*)mla::merge_out_uv_few<_Float16>
                                           : (const void*)mla::merge_out_uv_few<float>;
    st = launch("mla::merge_out_uv_few", k, dim3((unsigned)grid), dim3(256), a, s);
  } else if (w_dtype == MLA_BF16) {
    // workgroups per head: enough to fill the compute units, at most one per
    // 16-row tile
    const int tiles = (rows + 15) / 16;
    const int cus = device_cus() > 0 ? device_cus() : 256;
    a.groups = std::min(tiles, std::max(1, (cus + dims->heads - 1) / dims->heads));
    const int64_t grid = (int64_t)(dims->heads + 7) / 8 * 8 * a.groups;
    if (grid > 0x7fffffff) return MLA_ERR_SHAPE;
    const bool one = num_splits == 1;  // the single chunk: no first-round loads of absent chunks
    const void* k = part_dtype == MLA_F16
                        ? (one ? (const void*)mla::merge_out_uv16<_Float16, 1> : (const void*)mla::merge_out_uv16<_Float16, 4>)
                        : (one ? (const void*)mla::merge_out_uv16<float, 1> : (const void*)mla::merge_out_uv16<float, 4>);
    st = launch("mla::merge_out_uv16", k, dim3((unsigned)grid), dim3(256), a, s);
  } else {
    if (rows > 65535) return MLA_ERR_SHAPE;
    st = launch("mla::out_uv_f32<merge>", (const void*)mla::out_uv_f32<true>, dim3(dims->heads * (kDH / 16)),
                dim3(256), a, s);
  }
  return st;
}

namespace {

int append_chunks(int32_t d_model) { return (d_model + mla::kAppendChunk - 1) / mla::kAppendChunk; }

}  // namespace

int mla_cache_append_workspace_size(const mla_dims* dims, int32_t d_model, int64_t* bytes) {
  int st = check_dims(dims);
  if (st) return st;
  if (!bytes) return MLA_ERR_NULL;
  if (d_model < 64 || d_model > 65536 || d_model % 64) return MLA_ERR_SHAPE;
  *bytes = (int64_t)append_chunks(d_model) * dims->batch * dims->q_per_seq * mla::kAppendCols * 4;
  return MLA_OK;
}

}  // extern "C"

namespace {

// The shared body of mla_cache_append and mla_cache_append_static: with
// `workspace` NULL it validates only and stores the partial-sum bytes the
// call needs in *need (launching nothing).
int cache_append_impl(const mla_dims* dims, int32_t d_model, const void* h, const void* w_dkv, const void* w_kr,
                      int32_t in_dtype, float rope_theta, const mla_paged_kv* kv, void* workspace,
                      int64_t workspace_bytes, int64_t* need, void* stream) {
  int st = check_dims(dims);
  if (st) return st;
  if (!kv || !h || !w_dkv || !w_kr || (!workspace && !need)) return MLA_ERR_NULL;
  if (!kv->latent || !kv->rope || !kv->block_table || !kv->seq_lens) return MLA_ERR_NULL;
  if (d_model < 64 || d_model > 65536 || d_model % 64) return MLA_ERR_SHAPE;
  if (!(rope_theta > 0.f) || !isfinite(rope_theta)) return MLA_ERR_SHAPE;
  if (kv->block_size != kBlock || kv->num_blocks < 1 || kv->max_blocks_per_seq < 1) return MLA_ERR_SHAPE;
  const int32_t ld = kv->latent_dtype, rd = kv->rope_dtype;
  int fmt;  // 0 = f32, 1 = bf16, 2 = fp8
  if (in_dtype == MLA_F32 && ld == MLA_F32 && rd == MLA_F32) fmt = 0;
  else if (in_dtype == MLA_BF16 && ld == MLA_BF16 && rd == MLA_BF16) fmt = 1;
  else if (in_dtype == MLA_BF16 && ld == MLA_FP8_E4M3 && rd == MLA_BF16) fmt = 2;
  else return MLA_ERR_DTYPE;
  if (fmt == 2 && !kv->scale) return MLA_ERR_NULL;
  if (fmt != 2 && kv->scale) return MLA_ERR_DTYPE;
  if (kv->latent_row_stride < kDL || kv->rope_row_stride < kDR || kv->latent_block_stride < 0 ||
      kv->rope_block_stride < 0 || (fmt == 2 && kv->scale_block_stride < kBlock))
    return MLA_ERR_SHAPE;
  if (!aligned16(h) || !aligned16(w_dkv) || !aligned16(w_kr) || !aligned16(workspace)) return MLA_ERR_ALIGN;
  const int tokens = dims->batch * dims->q_per_seq;
  const int chunks = fmt == 0 ? 1 : append_chunks(d_model);
  if (!workspace) {
    *need = (int64_t)chunks * tokens * mla::kAppendCols * 4;
    return MLA_OK;
  }
  if (tokens == 0) return MLA_OK;
  if (workspace_bytes < (int64_t)chunks * tokens * mla::kAppendCols * 4) return MLA_ERR_SHAPE;
  if (check_mode()) {
    st = check_paging(dims->batch, kv, (hipStream_t)stream);
    if (st) return st;
  }
  const int64_t les = elem_size(ld), res = elem_size(rd);
  mla::AppendArgs a;
  a.h = h;
  a.w_dkv = w_dkv;
  a.w_kr = w_kr;
  a.part = (float*)workspace;
  a.latent = (uint8_t*)kv->latent;
  a.rope = (uint8_t*)kv->rope;
  a.scale = (float*)kv->scale;
  a.lat_bs = kv->latent_block_stride * les;
  a.lat_rs = kv->latent_row_stride * les;
  a.rope_bs = kv->rope_block_stride * res;
  a.rope_rs = kv->rope_row_stride * res;
  a.scale_bs = kv->scale_block_stride;
  a.block_table = kv->block_table;
  a.seq_lens = kv->seq_lens;
  a.tokens = tokens;
  a.sq = dims->q_per_seq;
  a.d_model = d_model;
  a.chunks = chunks;
  a.max_blocks = kv->max_blocks_per_seq;
  a.log2_theta = log2((double)rope_theta);
  hipStream_t s = (hipStream_t)stream;
  if (fmt == 0) {
    if (tokens > 65535) return MLA_ERR_SHAPE;
    st = launch("mla::append_proj_f32", (const void*)mla::append_proj_f32, dim3(mla::kAppendCols / 4, tokens),
                dim3(256), a, s);
  } else {
    const dim3 grid(mla::kAppendCols / 32, chunks, (tokens + 31) / 32);
    if (grid.z > 65535) return MLA_ERR_SHAPE;
    st = launch("mla::append_proj_mfma", (const void*)mla::append_proj_mfma, grid, dim3(256), a, s);
  }
  if (st) return st;
  if (fmt == 0)
    st = launch("mla::append_finish<f32>", (const void*)mla::append_finish<0>, dim3(tokens), dim3(256), a, s);
  else if (fmt == 1)
    st = launch("mla::append_finish<bf16>", (const void*)mla::append_finish<1>, dim3(tokens), dim3(256), a, s);
  else
    st = launch("mla::append_finish<fp8>", (const void*)mla::append_finish<2>, dim3(tokens), dim3(256), a, s);
  return st;
}

// ---- the no-allocation variant's scratch: one array per GPU, in this
// source's device code, for the fp32 chunk partial sums of the append.  Host
// code never passes `scratch` itself (its host-side name is not a device
// address): the device address is looked up once per device with that
// device current and kept in g_scratch.
constexpr int64_t kScratchBytes = MLA_STATIC_SCRATCH_BYTES;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices];

int scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MLA_ERR_DEVICE;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MLA_ERR_DEVICE;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return MLA_OK;
}

}  // namespace

extern "C" {

int mla_cache_append(const mla_dims* dims, int32_t d_model, const void* h, const void* w_dkv, const void* w_kr,
                     int32_t in_dtype, float rope_theta, const mla_paged_kv* kv, void* workspace,
                     int64_t workspace_bytes, void* stream) {
  if (!workspace) return MLA_ERR_NULL;
  return cache_append_impl(dims, d_model, h, w_dkv, w_kr, in_dtype, rope_theta, kv, workspace, workspace_bytes,
                           nullptr, stream);
}

int mla_cache_append_static(const mla_dims* dims, int32_t d_model, const void* h, const void* w_dkv,
                            const void* w_kr, int32_t in_dtype, float rope_theta, const mla_paged_kv* kv,
                            void* stream) {
  int64_t need = 0;
  int st = cache_append_impl(dims, d_model, h, w_dkv, w_kr, in_dtype, rope_theta, kv, nullptr, 0, &need, stream);
  if (st) return st;
  if (need > kScratchBytes) return MLA_ERR_SCRATCH;
  if (need == 0) return MLA_OK;
  void* ws = nullptr;
  st = scratch_address(&ws);
  if (st) return st;
  return cache_append_impl(dims, d_model, h, w_dkv, w_kr, in_dtype, rope_theta, kv, ws, kScratchBytes, nullptr,
                           stream);
}

namespace {

constexpr int32_t kGateMaxTokens = 65535 * 32;

// 0 on success.  The d_model slices of the affinity partial sums: their
// count in *chunks and width in *kslice (a multiple of 64; the last slice
// shorter).  bf16 inputs from kGateTallMinTokens tokens on take the tall
// kernel, with slices cut so that about 256 workgroups (one per compute
// unit) fill the device, none narrower than 512 unless d_model is; fewer
// tokens take 512-wide slices; fp32 inputs one slice.
int gate_shape(int32_t tokens, int32_t d_model, int32_t n_experts, int32_t in_dtype, int* chunks, int* kslice) {
  if (tokens < 0 || d_model < 64 || d_model > 65536 || d_model % 64 || n_experts < 1 ||
      n_experts > mla::kGateMaxExperts)
    return MLA_ERR_SHAPE;
  if (in_dtype == MLA_BF16) {
    if (tokens > kGateMaxTokens) return MLA_ERR_SHAPE;
    int ks = mla::kGateChunk;
    if (tokens >= mla::kGateTallMinTokens) {
      const int tiles = (tokens + mla::kGateTallM - 1) / mla::kGateTallM;
      const int want = std::max(1, std::min((256 + tiles - 1) / tiles, d_model / mla::kGateChunk));
      ks = ((d_model + want - 1) / want + 63) / 64 * 64;
    }
    *kslice = ks;
    *chunks = (d_model + ks - 1) / ks;
  } else if (in_dtype == MLA_F32) {
    if (tokens > 65535) return MLA_ERR_SHAPE;
    *kslice = d_model;
    *chunks = 1;
  } else {
    return MLA_ERR_DTYPE;
  }
  return MLA_OK;
}

}  // namespace

int mla_moe_gate_workspace_size(int32_t tokens, int32_t d_model, int32_t n_experts, int32_t in_dtype,
                                int64_t* bytes) {
  if (!bytes) return MLA_ERR_NULL;
  int chunks = 0, kslice = 0;
  const int st = gate_shape(tokens, d_model, n_experts, in_dtype, &chunks, &kslice);
  if (st) return st;
  *bytes = (int64_t)chunks * tokens * ((n_experts + 3) / 4 * 4) * 4;
  return MLA_OK;
}

int mla_moe_gate(int32_t tokens, int32_t d_model, int32_t n_experts, int32_t top_k, const void* u, const void* e,
                 int32_t in_dtype, int32_t* idx, float* weight, float* scores, void* workspace,
                 int64_t workspace_bytes, void* stream) {
  int chunks = 0, kslice = 0;
  int st = gate_shape(tokens, d_model, n_experts, in_dtype, &chunks, &kslice);
  if (st) return st;
  if (top_k < 1 || top_k > n_experts || top_k > mla::kGateMaxTopK) return MLA_ERR_SHAPE;
  if (tokens == 0) return MLA_OK;  // no token: nothing read or written, pointers unused
  if (!u || !e || !idx || !weight || !workspace) return MLA_ERR_NULL;
  if (!aligned16(u) || !aligned16(e) || !aligned16(workspace) || ((uintptr_t)idx & 3u) ||
      ((uintptr_t)weight & 3u) || ((uintptr_t)scores & 3u))
    return MLA_ERR_ALIGN;
  const int part_stride = (n_experts + 3) / 4 * 4;
  if (workspace_bytes < (int64_t)chunks * tokens * part_stride * 4) return MLA_ERR_SHAPE;
  mla::GateArgs a;
  a.u = u;
  a.e = e;
  a.part = (float*)workspace;
  a.idx = idx;
  a.weight = weight;
  a.scores = scores;
  a.tokens = tokens;
  a.d_model = d_model;
  a.n_experts = n_experts;
  a.top_k = top_k;
  a.chunks = chunks;
  a.kslice = kslice;
  a.part_stride = part_stride;
  hipStream_t s = (hipStream_t)stream;
  if (in_dtype == MLA_F32) {
    st = launch("mla::gate_proj_f32", (const void*)mla::gate_proj_f32, dim3((n_experts + 3) / 4, tokens), dim3(256),
                a, s);
  } else if (tokens >= mla::kGateTallMinTokens) {
    const dim3 grid(chunks, (tokens + mla::kGateTallM - 1) / mla::kGateTallM);
    const void* const tall[8] = {(const void*)mla::gate_proj_tall<1>, (const void*)mla::gate_proj_tall<2>,
                                 (const void*)mla::gate_proj_tall<3>, (const void*)mla::gate_proj_tall<4>,
                                 (const void*)mla::gate_proj_tall<5>, (const void*)mla::gate_proj_tall<6>,
                                 (const void*)mla::gate_proj_tall<7>, (const void*)mla::gate_proj_tall<8>};
    const void* k = tall[(n_experts + 31) / 32 - 1];
    st = launch("mla::gate_proj_tall", k, grid, dim3(256), a, s);
  } else {
    const dim3 grid((n_experts + 31) / 32, chunks, (tokens + 31) / 32);  // 32-expert tiles
    st = launch("mla::gate_proj_mfma", (const void*)mla::gate_proj_mfma, grid, dim3(256), a, s);
  }
  if (st) return st;
  if (tokens <= mla::kGateWideFinishMaxTokens)  // 64 lanes and up to 4 experts per lane per token
    return launch("mla::gate_finish<1, 64>", (const void*)mla::gate_finish<1, 64>, dim3((tokens + 3) / 4),
                  dim3(256), a, s);
  const void* const finish[4] = {(const void*)mla::gate_finish<1, 16>, (const void*)mla::gate_finish<2, 16>,
                                 (const void*)mla::gate_finish<3, 16>, (const void*)mla::gate_finish<4, 16>};
  return launch("mla::gate_finish", finish[(n_experts + 63) / 64 - 1], dim3((tokens + 15) / 16), dim3(256), a, s);
}

// Token capacity of the explicit form's workspace: the page table's span,
// rounded up to whole rebuild tiles.
static int64_t explicit_tokens(int32_t max_blocks_per_seq) {
  const int64_t t = (int64_t)max_blocks_per_seq * kBlock;
  return (t + mla::kRebuildTok - 1) / mla::kRebuildTok * mla::kRebuildTok;
}

int mla_attend_explicit_workspace_size(const mla_dims* dims, int32_t max_blocks_per_seq, int64_t* bytes) {
  int st = check_dims(dims);
  if (st) return st;
  if (!bytes) return MLA_ERR_NULL;
  if (max_blocks_per_seq < 1) return MLA_ERR_SHAPE;
  const int64_t tokens = explicit_tokens(max_blocks_per_seq);
  if (tokens > (1 << 24)) return MLA_ERR_SHAPE;
  *bytes = (int64_t)dims->batch * dims->heads * tokens * kDH * 2 * 2;  // K and V^T, bf16
  return MLA_OK;
}

int mla_attend_explicit(const mla_dims* dims, const void* q_nope, const void* q_rope, int32_t in_dtype,
                        const mla_paged_kv* kv, const void* w_uk, const void* w_uv, void* workspace,
                        int64_t workspace_bytes, void* out, int32_t out_dtype, float* lse, void* stream) {
  int st = check_dims(dims);
  if (st) return st;
  if (!kv || !q_nope || !q_rope || !w_uk || !w_uv || !workspace || !out) return MLA_ERR_NULL;
  if (!kv->latent || !kv->rope || !kv->block_table || !kv->seq_lens) return MLA_ERR_NULL;
  if (in_dtype != MLA_BF16 || kv->latent_dtype != MLA_BF16 || kv->rope_dtype != MLA_BF16 || kv->scale)
    return MLA_ERR_DTYPE;
  if (out_dtype != MLA_F32 && out_dtype != MLA_BF16) return MLA_ERR_DTYPE;
  if (kv->block_size != kBlock || kv->num_blocks < 1 || kv->max_blocks_per_seq < 1) return MLA_ERR_SHAPE;
  if (kv->latent_row_stride < kDL || kv->rope_row_stride < kDR || kv->latent_block_stride < 0 ||
      kv->rope_block_stride < 0)
    return MLA_ERR_SHAPE;
  // the kernels' per-lane copy offsets within a page are 32-bit
  if (kv->latent_row_stride > (1 << 24) || kv->rope_row_stride > (1 << 24)) return MLA_ERR_SHAPE;
  const int64_t lat_rs = kv->latent_row_stride * 2, lat_bs = kv->latent_block_stride * 2;
  const int64_t rope_rs = kv->rope_row_stride * 2, rope_bs = kv->rope_block_stride * 2;
  if (!aligned16(q_nope) || !aligned16(q_rope) || !aligned16(w_uk) || !aligned16(w_uv) || !aligned16(workspace) ||
      !aligned16(out) || !aligned16(kv->latent) || !aligned16(kv->rope) || (lat_rs & 15) || (lat_bs & 15) ||
      (rope_rs & 15) || (rope_bs & 15))
    return MLA_ERR_ALIGN;
  int64_t need = 0;
  st = mla_attend_explicit_workspace_size(dims, kv->max_blocks_per_seq, &need);
  if (st) return st;
  if (workspace_bytes < need) return MLA_ERR_SHAPE;
  if (dims->batch == 0) return MLA_OK;
  if (check_mode()) {
    st = check_paging(dims->batch, kv, (hipStream_t)stream);
    if (st) return st;
  }

  const int64_t tokens = explicit_tokens(kv->max_blocks_per_seq);
  mla::ExplicitArgs a;
  a.q_nope = (const uint16_t*)q_nope;
  a.q_rope = (const uint16_t*)q_rope;
  a.latent = (const uint8_t*)kv->latent;
  a.rope = (const uint8_t*)kv->rope;
  a.lat_bs = lat_bs;
  a.lat_rs = lat_rs;
  a.rope_bs = rope_bs;
  a.rope_rs = rope_rs;
  a.block_table = kv->block_table;
  a.seq_lens = kv->seq_lens;
  a.w_uk = (const uint16_t*)w_uk;
  a.w_uv = (const uint16_t*)w_uv;
  a.k = (uint16_t*)workspace;
  a.vt = (uint16_t*)workspace + (int64_t)dims->batch * dims->heads * tokens * kDH;
  a.out = out;
  a.lse = lse;
  a.batch = dims->batch;
  a.sq = dims->q_per_seq;
  a.heads = dims->heads;
  a.max_blocks = kv->max_blocks_per_seq;
  a.tokens = (int)tokens;
  a.tiles = (int)(tokens / mla::kRebuildTok);
  a.qblocks = (dims->q_per_seq + mla::kExplicitQ - 1) / mla::kExplicitQ;
  a.out_bf16 = out_dtype == MLA_BF16;
  a.scale_log2 = dims->softmax_scale * 1.4426950408889634f;
  // grids: a multiple of the 8 XCDs over the (token tile, head) blocks and
  // the ((sequence, head), query block) items -- see the kernels' placement
  const int64_t rb_items = ((int64_t)dims->batch * a.tiles + mla::kRbBlockT - 1) / mla::kRbBlockT *
                           ((dims->heads + mla::kRbBlockH - 1) / mla::kRbBlockH) * mla::kRbBlockT * mla::kRbBlockH;
  const int64_t rb_grid = (rb_items + 7) / 8 * 8;
  const int64_t at_grid = 8 * (((int64_t)dims->batch * dims->heads + 7) / 8) * a.qblocks;
  if (rb_grid > 0x7fffffff || at_grid > 0x7fffffff) return MLA_ERR_SHAPE;
  hipStream_t s = (hipStream_t)stream;
  st = launch("mla::rebuild_kv", (const void*)mla::rebuild_kv, dim3((unsigned)rb_grid), dim3(512), a, s);
  if (st) return st;
  return launch("mla::attend_explicit", (const void*)mla::attend_explicit, dim3((unsigned)at_grid), dim3(64 * mla::kAtWaves),
                a, s);
}

int mla_attention_form(const mla_dims* dims, int32_t latent_dtype, int32_t* form) {
  int st = check_dims(dims);
  if (st) return st;
  if (!form) return MLA_ERR_NULL;
  if (latent_dtype != MLA_F32 && latent_dtype != MLA_BF16 && latent_dtype != MLA_FP8_E4M3) return MLA_ERR_DTYPE;
  *form = latent_dtype == MLA_BF16 && dims->q_per_seq >= MLA_EXPLICIT_MIN_Q ? MLA_FORM_EXPLICIT : MLA_FORM_ABSORBED;
  return MLA_OK;
}

// Pages per chunk an uneven batch is cut for (the headline's chunks: 4096
// tokens in 4).
constexpr int kRaggedChunkPages = 16;

int mla_decode_num_splits_batch(const mla_dims* dims, int64_t total_tokens, int32_t max_seq_len,
                                int32_t* num_splits) {
  int st = check_dims(dims);
  if (st) return st;
  if (!num_splits) return MLA_ERR_NULL;
  if (total_tokens < 0 || max_seq_len < 0 || total_tokens > (int64_t)dims->batch * max_seq_len) return MLA_ERR_SHAPE;
  int32_t ns = 1;
  st = mla_decode_num_splits(dims, max_seq_len, &ns);
  if (st) return st;
  const int64_t b = dims->batch;
  if (b >= 2 && total_tokens * 10 < b * (int64_t)max_seq_len * 9) {  // uneven lengths
    const int64_t mean_pages = ((total_tokens + kBlock - 1) / kBlock + b - 1) / b;
    const int64_t max_pages = ((int64_t)max_seq_len + kBlock - 1) / kBlock;
    int64_t want = (mean_pages + kRaggedChunkPages / 2) / kRaggedChunkPages;
    if (want > max_pages) want = max_pages;
    if (want > MLA_MAX_SPLITS) want = MLA_MAX_SPLITS;
    if (want > ns) ns = (int32_t)want;
  }
  *num_splits = ns;
  return MLA_OK;
}

int mla_decode_num_splits(const mla_dims* dims, int32_t max_seq_len, int32_t* num_splits) {
  int st = check_dims(dims);
  if (st) return st;
  if (!num_splits) return MLA_ERR_NULL;
  if (max_seq_len < 0) return MLA_ERR_SHAPE;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
    return MLA_ERR_DEVICE;
  const int rows = dims->q_per_seq * dims->heads;
  const int64_t per_split = (int64_t)(dims->batch > 0 ? dims->batch : 1) *
                            ((rows + mla::kDecodeRowsPerWg - 1) / mla::kDecodeRowsPerWg);
  const int pages = (max_seq_len + kBlock - 1) / kBlock;
  int64_t ns = (cus + per_split - 1) / per_split;
  // keep at least 4 pages (256 tokens) per chunk so each workgroup streams
  // enough, except with few query rows (below one 64-row block per
  // sequence), where a page per chunk spreads a small problem over more
  // compute units
  const int min_pages = rows >= mla::kDecodeRowsPerWg ? 4 : 1;
  const int64_t max_ns = pages / min_pages > 0 ? pages / min_pages : 1;
  if (ns > max_ns) ns = max_ns;
  if (ns > MLA_MAX_SPLITS) ns = MLA_MAX_SPLITS;
  if (ns < 1) ns = 1;
  *num_splits = (int32_t)ns;
  return MLA_OK;
}

}  // extern "C"
