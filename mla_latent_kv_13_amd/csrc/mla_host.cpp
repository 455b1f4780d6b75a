// Host-only half of the MLA decode library: argument validation, workspace
// sizing, the split-count / page-size heuristic and status strings.  Nothing
// here calls the HIP runtime or touches device memory, so all of it runs (and
// is tested) on a machine without a GPU.
#include <cstddef>
#include <cstdint>

#include "mla_decode.h"

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool supported_pair(int32_t qd, int32_t kd) {
  if (kd == MLA_DTYPE_BF16) return qd == MLA_DTYPE_BF16;
  if (kd == MLA_DTYPE_FP8_E4M3FN)
    return qd == MLA_DTYPE_BF16 || qd == MLA_DTYPE_FP8_E4M3FN || qd == MLA_Q_BF16_FP8_STATIC;
  if (kd == MLA_DTYPE_MXFP4) return qd == MLA_DTYPE_BF16 || qd == MLA_DTYPE_MXFP4 || qd == MLA_Q_BF16_MXFP4;
  return false;
}

// KV bytes per cache row (scales included) - the dominant stream of stage 1.
int64_t kv_row_bytes(int32_t kd) {
  switch (kd) {
    case MLA_DTYPE_BF16: return 2 * MLA_HEAD_DIM_QK;
    case MLA_DTYPE_FP8_E4M3FN: return MLA_HEAD_DIM_QK;
    case MLA_KV_MXFP4_K_FP8_V: return MLA_MXFP4_ROW_BYTES + MLA_MXFP4_ROW_SCALES + MLA_HEAD_DIM_V;
    default: return MLA_MXFP4_ROW_BYTES + MLA_MXFP4_ROW_SCALES;
  }
}

}  // namespace

namespace {
// Measured fastest (split count, page size) on the 8-shape grid for every
// (Q, cache) format pair, written by mla_latent_kv_13_amd/tune.py, with the
// cost models' own picks and their measured time beside each (a record of
// how close the fallback models are).
struct TuneEntry {
  int32_t batch, kv_len, q_dtype, kv_dtype, splits, page_size;
  double us;
  int32_t model_splits, model_page_size;
  double model_us;
};
constexpr TuneEntry kTuneTable[] = {
#include "tune_table.inc"
};

// The tuned entry of a grid shape on a 256-CU device (MI355X), or NULL.
const TuneEntry* tuned(int32_t batch, int32_t kv_len, int32_t q_dtype, int32_t kv_dtype, int32_t num_cus) {
  if (num_cus != 256) return nullptr;
  for (const TuneEntry& e : kTuneTable)
    if (e.batch == batch && e.kv_len == kv_len && e.q_dtype == q_dtype && e.kv_dtype == kv_dtype) return &e;
  return nullptr;
}

// bf16 Q quantised in the call runs the fp8-Q or mxfp4-Q kernel: it takes
// that format's picks
int32_t valid_q(int32_t q) {
  if (q == MLA_Q_BF16_FP8_STATIC) return MLA_DTYPE_FP8_E4M3FN;
  if (q == MLA_Q_BF16_MXFP4) return MLA_DTYPE_MXFP4;
  return q == MLA_DTYPE_FP8_E4M3FN || q == MLA_DTYPE_MXFP4 ? q : MLA_DTYPE_BF16;
}
int32_t valid_kv(int32_t kv) { return kv < MLA_DTYPE_BF16 || kv > MLA_KV_MXFP4_K_FP8_V ? MLA_DTYPE_FP8_E4M3FN : kv; }
}  // namespace

extern "C" {

int32_t mla_abi_version(void) { return MLA_ABI_VERSION; }

const char* mla_status_string(int status) {
  switch (status) {
    case MLA_OK: return "ok";
    case MLA_ERR_NULL: return "a required pointer is NULL";
    case MLA_ERR_DTYPE: return "unsupported (q, kv) element format pair";
    case MLA_ERR_ARG: return "a size or count is out of range";
    case MLA_ERR_ALIGN: return "a buffer is not 16-byte aligned";
    case MLA_ERR_WORKSPACE: return "workspace missing or too small";
    case MLA_ERR_LAUNCH: return "the HIP runtime rejected a kernel launch";
    case MLA_ERR_DEVICE: return "no usable gfx950 device";
    default: return "unknown status";
  }
}

namespace {
// partial outputs (16-byte aligned rows), then the log-sum-exps, for `parts`
// partial rows of 512 values
size_t workspace_for_parts(size_t parts) { return parts * MLA_HEAD_DIM_V * sizeof(float) + parts * sizeof(float); }
}  // namespace

size_t mla_workspace_bytes_rows(int32_t batch, int32_t q_rows, int32_t num_splits) {
  if (q_rows < MLA_NUM_HEADS || q_rows % MLA_NUM_HEADS || q_rows > MLA_MAX_Q_ROWS) return 0;
  if (batch < 1 || num_splits < 1 || num_splits > MLA_MAX_SPLITS) return 0;
  if (num_splits == 1) return 0;
  return workspace_for_parts(static_cast<size_t>(batch) * static_cast<size_t>(num_splits) * q_rows);
}

size_t mla_workspace_bytes(int32_t batch, int32_t num_splits) {
  return mla_workspace_bytes_rows(batch, MLA_NUM_HEADS, num_splits);
}

int mla_validate(const void* q, int32_t q_dtype, const void* q_scale, const void* kv_cache,
                 int32_t kv_dtype, const void* kv_scale, int64_t num_kv_rows,
                 const int32_t* kv_indptr, int32_t batch, const int32_t* page_table,
                 const int32_t* page_indptr, int32_t page_size, int32_t num_splits, void* out,
                 void* workspace, size_t workspace_bytes) {
  (void)page_indptr;  // optional
  if (batch < 0) return MLA_ERR_ARG;
  if (page_size < 1 || num_splits < 1 || num_splits > MLA_MAX_SPLITS) return MLA_ERR_ARG;
  // rows are indexed with 32-bit arithmetic on the device
  if (num_kv_rows < 0 || num_kv_rows > 0xffffffffLL) return MLA_ERR_ARG;
  if (static_cast<int64_t>(batch) * num_splits > 0x7fffffffLL) return MLA_ERR_ARG;
  if (!supported_pair(q_dtype, kv_dtype)) return MLA_ERR_DTYPE;
  if (batch == 0) return MLA_OK;  // nothing to do
  if (!q || !kv_cache || !kv_indptr || !page_table || !out) return MLA_ERR_NULL;
  if (q_dtype != MLA_DTYPE_BF16 && q_dtype != MLA_Q_BF16_MXFP4 && !q_scale) return MLA_ERR_NULL;
  if (kv_dtype != MLA_DTYPE_BF16 && !kv_scale) return MLA_ERR_NULL;
  if (num_kv_rows < 1) return MLA_ERR_ARG;
  if (!aligned16(q) || !aligned16(kv_cache) || !aligned16(out)) return MLA_ERR_ALIGN;
  if (kv_dtype == MLA_DTYPE_MXFP4 && !aligned16(kv_scale)) return MLA_ERR_ALIGN;
  if (kv_dtype == MLA_DTYPE_FP8_E4M3FN && (reinterpret_cast<uintptr_t>(kv_scale) & 3u)) return MLA_ERR_ALIGN;
  if ((q_dtype == MLA_DTYPE_FP8_E4M3FN || q_dtype == MLA_Q_BF16_FP8_STATIC) &&
      (reinterpret_cast<uintptr_t>(q_scale) & 3u))
    return MLA_ERR_ALIGN;
  const size_t need = mla_workspace_bytes(batch, num_splits);
  if (need) {
    if (!workspace || workspace_bytes < need) return MLA_ERR_WORKSPACE;
    if (!aligned16(workspace)) return MLA_ERR_ALIGN;
  }
  return MLA_OK;
}

int mla_validate_mixed(const void* q, int32_t q_dtype, const void* q_scale, int32_t q_rows, const void* k_cache,
                       const void* k_scale, const void* v_cache, const void* v_scale, int64_t num_kv_rows,
                       const int32_t* kv_indptr, int32_t batch, const int32_t* page_table,
                       const int32_t* page_indptr, int32_t page_size, int32_t num_splits, void* out,
                       void* workspace, size_t workspace_bytes) {
  if (q_rows < MLA_NUM_HEADS || q_rows % MLA_NUM_HEADS || q_rows > MLA_MAX_Q_ROWS) return MLA_ERR_ARG;
  // Q is bf16 or mxfp4 (no in-call quantisation over the split cache)
  if (q_dtype != MLA_DTYPE_BF16 && q_dtype != MLA_DTYPE_MXFP4) return MLA_ERR_DTYPE;
  // the K side is an mxfp4 cache in every respect; its workspace check is
  // for 16 rows, so it is redone below for q_rows
  int rc = mla_validate(q, q_dtype, q_scale, k_cache, MLA_DTYPE_MXFP4, k_scale, num_kv_rows, kv_indptr, batch,
                        page_table, page_indptr, page_size, num_splits, out, nullptr, 0);
  if (rc == MLA_ERR_WORKSPACE) rc = MLA_OK;
  if (rc != MLA_OK || batch == 0) return rc;
  if (!v_cache || !v_scale) return MLA_ERR_NULL;
  if (!aligned16(v_cache) || (reinterpret_cast<uintptr_t>(v_scale) & 3u)) return MLA_ERR_ALIGN;
  const size_t need = mla_workspace_bytes_rows(batch, q_rows, num_splits);
  if (need) {
    if (!workspace || workspace_bytes < need) return MLA_ERR_WORKSPACE;
    if (!aligned16(workspace)) return MLA_ERR_ALIGN;
  }
  return MLA_OK;
}

int mla_check_tables(const int32_t* kv_indptr_host, int32_t batch, const int32_t* page_table_host,
                     int64_t page_table_len, const int32_t* page_indptr_host, int32_t page_size,
                     int64_t num_kv_rows, int32_t* bad_request) {
  if (bad_request) *bad_request = -1;
  if (batch < 0 || page_size < 1 || page_table_len < 0 || num_kv_rows < 0) return MLA_ERR_ARG;
  if (!kv_indptr_host) return MLA_ERR_NULL;
  if (page_table_len > 0 && !page_table_host) return MLA_ERR_NULL;
  if (kv_indptr_host[0] < 0) return MLA_ERR_ARG;
  const int64_t P = page_size;
  for (int32_t b = 0; b < batch; ++b) {
    const int64_t g0 = kv_indptr_host[b], g1 = kv_indptr_host[b + 1];
    auto fail = [&]() {
      if (bad_request) *bad_request = b;
      return MLA_ERR_ARG;
    };
    if (g1 < g0) return fail();
    if (g1 == g0) continue;
    // token t sits at position p = p0 + t of the table stream: entry p / P,
    // row offset p % P inside that page (one shared table: p0 = g0; per
    // request tables: p0 = page_indptr[b] * P)
    int64_t p0 = g0;
    if (page_indptr_host) {
      if (page_indptr_host[b] < 0) return fail();
      p0 = static_cast<int64_t>(page_indptr_host[b]) * P;
    }
    const int64_t p1 = p0 + (g1 - g0);
    for (int64_t j = p0 / P; j <= (p1 - 1) / P; ++j) {
      if (j >= page_table_len) return fail();
      const int64_t pid = page_table_host[j];
      // highest in-page offset this request uses on page j
      const int64_t hi = (p1 - 1 < j * P + P - 1 ? p1 - 1 : j * P + P - 1) - j * P;
      if (pid < 0 || pid * P + hi >= num_kv_rows) return fail();
    }
  }
  return MLA_OK;
}

int32_t mla_choose_num_splits(int32_t batch, int32_t kv_len, int32_t q_dtype, int32_t kv_dtype, int32_t num_cus) {
  if (batch < 1 || kv_len < 1) return 1;
  if (num_cus <= 0) num_cus = 256;
  q_dtype = valid_q(q_dtype);
  kv_dtype = valid_kv(kv_dtype);
  // Shapes of the tuned grid (MI355X, 256 CUs) take the measured optimum.
  if (const TuneEntry* e = tuned(batch, kv_len, q_dtype, kv_dtype, num_cus)) return e->splits;
  // Cost in "bytes streamed by the busiest CU": stage 1 runs in
  // ceil(batch*S / num_cus) rounds of one workgroup per CU, each streaming
  // its chunk rounded up to 128 tokens (four waves x 32-token sub-tiles);
  // S > 1 adds the partial outputs (written and re-read, spread over the
  // CUs), a fixed second launch worth ~3 us of per-CU bandwidth, and ~0.12 us
  // of stage-2 latency per split (its split loop), as measured on the grid.
  // mxfp4 tiles take as long to compute as fp8 ones (the e2m1 -> bf16 work
  // for P*V), so they are priced like a 576-byte fp8 row, not by their bytes
  const double row = static_cast<double>(kv_dtype == MLA_DTYPE_MXFP4 ? MLA_HEAD_DIM_QK : kv_row_bytes(kv_dtype));
  const double cu_bytes_per_us = 8.0e12 / 256.0 * 1e-6;
  const double launch_bytes = 3.0 * cu_bytes_per_us;
  const double per_split_bytes = 0.12 * cu_bytes_per_us;
  const int32_t max_s = kv_len / 32 < 1 ? 1 : (kv_len / 32 > MLA_MAX_SPLITS ? MLA_MAX_SPLITS : kv_len / 32);
  double best = 0.0;
  int32_t best_s = 1;
  for (int32_t s = 1; s <= max_s; ++s) {
    const int64_t chunk = (static_cast<int64_t>(kv_len) + s - 1) / s;
    const int64_t chunk_eff = (chunk + 127) / 128 * 128;
    const int64_t rounds = (static_cast<int64_t>(batch) * s + num_cus - 1) / num_cus;
    double cost = static_cast<double>(rounds) * static_cast<double>(chunk_eff) * row;
    if (s > 1) {
      const double partial = static_cast<double>(batch) * s * MLA_NUM_HEADS * (MLA_HEAD_DIM_V + 1) * 4.0 * 2.0;
      cost += partial / num_cus + launch_bytes + per_split_bytes * s;
    }
    if (s == 1 || cost < best * 0.999) {
      best = cost;
      best_s = s;
    }
  }
  return best_s;
}

int mla_plan_worklist(const int32_t* kv_indptr_host, int32_t batch, int32_t num_cus, int32_t max_items,
                      int32_t* items_host, int32_t* req_host, int32_t* num_items, int32_t* num_slots) {
  if (!num_items || !num_slots) return MLA_ERR_NULL;
  *num_items = 0;
  *num_slots = 0;
  if (batch < 0 || max_items < batch) return MLA_ERR_ARG;
  if (batch == 0) return MLA_OK;
  if (!kv_indptr_host || !items_host || !req_host) return MLA_ERR_NULL;
  if (num_cus <= 0) num_cus = 256;
  int64_t total = 0;
  for (int32_t b = 0; b < batch; ++b) {
    const int64_t L = static_cast<int64_t>(kv_indptr_host[b + 1]) - kv_indptr_host[b];
    if (L < 0) return MLA_ERR_ARG;
    total += L;
  }
  // Aim at whole rounds of one workgroup per CU: the smallest chunk (a
  // multiple of 128 tokens, at least 256) whose items fit ceil(batch /
  // num_cus) rounds; each extra round would pay the per-workgroup prologue
  // and epilogue again.
  int64_t max_len = 0;
  for (int32_t b = 0; b < batch; ++b) {
    const int64_t L = static_cast<int64_t>(kv_indptr_host[b + 1]) - kv_indptr_host[b];
    if (L > max_len) max_len = L;
  }
  const int64_t target = ((static_cast<int64_t>(batch) + num_cus - 1) / num_cus) * num_cus;
  auto count_items = [&](int64_t c) {
    int64_t n = 0;
    for (int32_t b = 0; b < batch; ++b) {
      const int64_t L = static_cast<int64_t>(kv_indptr_host[b + 1]) - kv_indptr_host[b];
      n += L > 0 ? (L + c - 1) / c : 1;
    }
    return n;
  };
  int64_t chunk = (total + target - 1) / target;
  chunk = (chunk + 127) / 128 * 128;
  if (chunk < 256) chunk = 256;
  while (chunk < max_len && count_items(chunk) > target) chunk = (chunk + chunk / 8 + 127) / 128 * 128;
  while (count_items(chunk) > max_items) chunk *= 2;
  int32_t ni = 0, ns = 0;
  for (int32_t b = 0; b < batch; ++b) {
    const int64_t L = static_cast<int64_t>(kv_indptr_host[b + 1]) - kv_indptr_host[b];
    const int64_t n = L > 0 ? (L + chunk - 1) / chunk : 1;
    req_host[2 * b] = n > 1 ? ns : -1;
    req_host[2 * b + 1] = static_cast<int32_t>(n);
    for (int64_t j = 0; j < n; ++j) {
      // item j covers [floor(jL/n), floor((j+1)L/n)): sizes differ by at most
      // one token and none is empty (n <= L)
      const int64_t t0 = j * L / n;
      const int64_t cnt = (j + 1) * L / n - t0;
      int32_t* it = items_host + 4 * ni;
      it[0] = b;
      it[1] = static_cast<int32_t>(t0);
      it[2] = static_cast<int32_t>(cnt);
      it[3] = n > 1 ? ns++ : -1;
      ++ni;
    }
  }
  *num_items = ni;
  *num_slots = ns;
  return MLA_OK;
}

size_t mla_worklist_workspace_bytes(int32_t num_slots, int32_t q_rows) {
  if (num_slots <= 0 || q_rows < MLA_NUM_HEADS || q_rows % MLA_NUM_HEADS || q_rows > MLA_MAX_Q_ROWS) return 0;
  return workspace_for_parts(static_cast<size_t>(num_slots) * q_rows);
}

int32_t mla_recommend_page_size(int32_t batch, int32_t kv_len, int32_t q_dtype, int32_t kv_dtype, int32_t num_cus) {
  if (batch < 1 || kv_len < 1) return 1;
  if (num_cus <= 0) num_cus = 256;
  q_dtype = valid_q(q_dtype);
  kv_dtype = valid_kv(kv_dtype);
  if (const TuneEntry* e = tuned(batch, kv_len, q_dtype, kv_dtype, num_cus)) return e->page_size;
  // Model: pages long enough that a 32-token sub-tile gathers few separate
  // runs (each DMA instruction then reads long contiguous runs of rows and
  // the table costs one 4-byte id per page), but no longer than a quarter of
  // a request, so a request's last page wastes little of the cache.
  int32_t p = 1;
  while (p < 16 && 4 * (2 * p) <= kv_len) p *= 2;
  return p;
}

}  // extern "C"
