// C-ABI host layer of libsma: argument checks, launch planning and kernel
// launches on the caller's stream. No allocation, no synchronization.
//
// Conventions carried over from the backend pages: sizes and raw device
// pointers at the boundary (oxicuda ComputeBackend `attention`), status codes
// rather than exceptions (its BackendResult / BackendError::Unsupported),
// outputs that must not alias inputs (pulsatrix HIPBackend `gemm_ex`), and an
// idempotent lazily filled device cache (oxicuda `init`).
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <mutex>

#include "sma.h"
#include "sma_kernels.h"

namespace {

constexpr size_t kMaxSeq = size_t(1) << 30;     // keeps the kernels' int32 key/row math exact
constexpr size_t kMaxWorkgroups = (size_t(1) << 32) / sma::kThreadsPerWG - 1;
constexpr int kMaxSplits = 32;
constexpr size_t kWsAlign = 256;

struct Shape {
  int in_dtype, o_dtype;
  int layout;                            // SMA_LAYOUT_*
  size_t batch, heads, seq_q, seq_kv, d;
  size_t row_elems;                      // elements between consecutive rows of one head
  size_t bh, rows;                       // batch*heads, batch*heads*seq_q
  size_t q_bytes, kv_bytes, o_bytes, lse_bytes;
  bool masked;                           // a hard mask (the 16-bit kernel at head dim 128 differs)
};

bool mul(size_t a, size_t b, size_t* out) {
  if (a != 0 && b > SIZE_MAX / a) return false;
  *out = a * b;
  return true;
}

size_t elem_bytes(int dt) { return dt == SMA_DTYPE_F32 ? 4 : 2; }

// Checks that do not depend on pointers. Fills sh on success.
int check_shape(int in_dtype, int o_dtype, size_t batch, size_t heads, size_t seq_q, size_t seq_kv,
                size_t d, double scale, Shape* sh, int layout = SMA_LAYOUT_BHSD) {
  if (layout != SMA_LAYOUT_BHSD && layout != SMA_LAYOUT_BSHD) return SMA_ERR_INVALID_VALUE;
  if (in_dtype != SMA_DTYPE_F32 && in_dtype != SMA_DTYPE_BF16 && in_dtype != SMA_DTYPE_F16)
    return SMA_ERR_INVALID_VALUE;
  if (o_dtype != SMA_DTYPE_F32 && o_dtype != SMA_DTYPE_BF16 && o_dtype != SMA_DTYPE_F16)
    return SMA_ERR_INVALID_VALUE;
  if (d == 0) return SMA_ERR_INVALID_VALUE;
  if (!std::isfinite(scale)) return SMA_ERR_INVALID_VALUE;
  Shape s{};
  s.in_dtype = in_dtype;
  s.o_dtype = o_dtype;
  s.layout = layout;
  s.batch = batch;
  s.heads = heads;
  s.seq_q = seq_q;
  s.seq_kv = seq_kv;
  s.d = d;
  size_t nq, nkv, t;
  if (!mul(batch, heads, &s.bh) || !mul(s.bh, seq_q, &s.rows) || !mul(s.rows, d, &nq) ||
      !mul(s.bh, seq_kv, &t) || !mul(t, d, &nkv) || !mul(nq, elem_bytes(in_dtype), &s.q_bytes) ||
      !mul(nkv, elem_bytes(in_dtype), &s.kv_bytes) || !mul(nq, elem_bytes(o_dtype), &s.o_bytes) ||
      !mul(s.rows, sizeof(float), &s.lse_bytes))
    return SMA_ERR_INVALID_VALUE;
  // Head dims 32, 64 and 128 run on every kernel; 256 on the query-block
  // kernels (fp32 and 16-bit), not on the fp32 in-workgroup key-split one.
  if (d != 32 && d != 64 && d != 128 && d != 256) return SMA_ERR_UNSUPPORTED;
  if (seq_q > kMaxSeq || seq_kv > kMaxSeq || s.bh > (size_t(1) << 31)) return SMA_ERR_UNSUPPORTED;
  if (heads > (size_t(1) << 20)) return SMA_ERR_UNSUPPORTED;
  s.row_elems = layout == SMA_LAYOUT_BSHD ? heads * d : d;
  // The 16-bit kernel addresses one (batch, head)'s K and V through 32-bit
  // buffer offsets: keep them, with a tile of slack, below 2^31 bytes.
  if (in_dtype != SMA_DTYPE_F32 && (seq_kv + 256) * s.row_elems * 2 > (size_t(1) << 31))
    return SMA_ERR_UNSUPPORTED;
  *sh = s;
  return SMA_OK;
}

struct Plan {
  int kernel = SMA_KERNEL_F32_QBLOCK;
  int32_t nqb = 0, nsplit = 1, split_len = 0;
  size_t nwg = 0;
  size_t ws_bytes = 0;       // workspace the split needs (0 when nsplit == 1)
  size_t part_lse_off = 0;   // byte offset of the partial LSE array in the workspace
};

// The 16-bit kernel at head dim 128 takes two 32-row blocks per wave (512 rows, 32-key
// tiles) without a hard mask; with one it runs the 32-row kernel of the other head dims,
// whose 64-key tiles read the mask's column words half as often per key.
int queries_per_wg(int kernel, const Shape& s) {
  switch (kernel) {
    case SMA_KERNEL_F32_KSPLIT: return sma::kF32WsplitQueriesPerWG;
    case SMA_KERNEL_BF16_QBLOCK:
      return s.d == 256 ? sma::kBF16D256QueriesPerWG
             : s.d == 128 && !s.masked ? sma::kBF16D128QueriesPerWG : sma::kBF16QueriesPerWG;
    default: return sma::kF32QueriesPerWG;
  }
}
int keys_per_tile(int kernel, const Shape& s) {
  if (kernel == SMA_KERNEL_BF16_QBLOCK)
    return s.d == 256 ? sma::kBF16D256KeysPerTile
           : s.d == 128 && !s.masked ? sma::kBF16D128KeysPerTile : sma::kBF16KeysPerTile;
  return sma::kF32KeysPerTile;
}
bool kernel_fits_dtype(int kernel, int in_dtype) {
  if (in_dtype != SMA_DTYPE_F32) return kernel == SMA_KERNEL_BF16_QBLOCK;
  return kernel == SMA_KERNEL_F32_QBLOCK || kernel == SMA_KERNEL_F32_KSPLIT;
}

size_t round_up(size_t x, size_t m) { return (x + m - 1) / m * m; }

// Key splits for a query-block kernel when its blocks alone cannot fill the
// GPU: aim for one resident workgroup per slot, keep at least four key tiles
// per split.
size_t auto_splits(const Shape& s, int kernel, size_t base, int num_cus) {
  const size_t kt = (size_t)keys_per_tile(kernel, s);
  // Resident workgroups per CU: one for the 16-bit kernel and for head dim 256
  // (LDS-limited), two otherwise.
  const size_t per_cu = kernel == SMA_KERNEL_BF16_QBLOCK || s.d > 128 ? 1 : 2;
  const size_t slots = (size_t)num_cus * per_cu;
  size_t nsplit = 1;
  if (base > 0 && base < slots && s.seq_kv >= 8 * kt) {
    size_t want = (slots + base - 1) / base;
    size_t by_keys = s.seq_kv / (4 * kt);
    nsplit = want < by_keys ? want : by_keys;
    if (nsplit > (size_t)kMaxSplits) nsplit = kMaxSplits;
    if (nsplit < 1) nsplit = 1;
  }
  return nsplit;
}

// The fp32 kernel that splits keys over the waves of one 32-row workgroup
// needs no workspace and no second launch, and measures faster than the
// 128-row kernel on every shape whose 32-row grid fills the GPU (short and
// long key ranges alike). With fewer 32-row blocks than CUs and long rows
// (decode-like shapes), the 128-row kernel with a key split across
// workgroups keeps more of the GPU busy.
constexpr size_t kKsplitAlwaysKeys = 512;

// The in-workgroup key-split kernel addresses one (batch, head)'s Q, K and V
// through 32-bit buffer offsets: keep them, with a tile of slack, below 2^31.
bool ksplit_fits(const Shape& s) {
  const size_t lim = size_t(1) << 31;
  return (s.seq_q + 32) * s.row_elems * 4 <= lim && (s.seq_kv + 32) * s.row_elems * 4 <= lim;
}

// Kernels built for a head dim (the query-block kernels also for 256: the
// in-workgroup key-split kernel's per-wave K and V slots would not fit LDS).
bool kernel_fits_head_dim(int kernel, size_t d) {
  return d != 256 || kernel == SMA_KERNEL_F32_QBLOCK || kernel == SMA_KERNEL_BF16_QBLOCK;
}

int auto_kernel(const Shape& s, int num_cus) {
  if (s.in_dtype != SMA_DTYPE_F32) return SMA_KERNEL_BF16_QBLOCK;
  if (!ksplit_fits(s) || !kernel_fits_head_dim(SMA_KERNEL_F32_KSPLIT, s.d)) return SMA_KERNEL_F32_QBLOCK;
  const size_t nwg32 = s.bh * ((s.seq_q + sma::kF32WsplitQueriesPerWG - 1) / sma::kF32WsplitQueriesPerWG);
  if (nwg32 >= (size_t)num_cus || s.seq_kv <= kKsplitAlwaysKeys) return SMA_KERNEL_F32_KSPLIT;
  return SMA_KERNEL_F32_QBLOCK;
}

// Plan for `kernel` with `nsplit` key splits (0: chosen here). The caller has
// checked that the kernel fits the dtype and that nsplit is in range.
Plan plan_for(const Shape& s, int kernel, size_t nsplit, int num_cus) {
  Plan p;
  p.kernel = kernel;
  const size_t qpw = (size_t)queries_per_wg(kernel, s);
  const size_t kt = (size_t)keys_per_tile(kernel, s);
  p.nqb = (int32_t)((s.seq_q + qpw - 1) / qpw);
  const size_t base = s.bh * (size_t)p.nqb;
  if (kernel == SMA_KERNEL_F32_KSPLIT || s.seq_kv == 0) nsplit = 1;
  if (nsplit == 0) nsplit = auto_splits(s, kernel, base, num_cus);
  size_t split_len = s.seq_kv;
  if (nsplit > 1) {
    split_len = round_up((s.seq_kv + nsplit - 1) / nsplit, kt);
    nsplit = (s.seq_kv + split_len - 1) / split_len;
  }
  if (split_len == 0) split_len = kt;
  if (nsplit < 1) nsplit = 1;
  p.nsplit = (int32_t)nsplit;
  p.split_len = (int32_t)split_len;
  p.nwg = base * nsplit;
  if (nsplit > 1) {
    const size_t part_o = nsplit * s.rows * s.d * sizeof(float);
    p.part_lse_off = round_up(part_o, kWsAlign);
    p.ws_bytes = p.part_lse_off + round_up(nsplit * s.rows * sizeof(float), kWsAlign);
  }
  return p;
}

Plan auto_plan(const Shape& s, int num_cus) { return plan_for(s, auto_kernel(s, num_cus), 0, num_cus); }

bool overlap(const void* a, size_t na, const void* b, size_t nb) {
  if (!a || !b || na == 0 || nb == 0) return false;
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + nb && y < x + na;
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

int check_pointers(const Shape& s, const void* q, const void* k, const void* v, const void* o,
                   const float* lse, const void* ws, size_t ws_bytes) {
  if (!q || !o) return SMA_ERR_NULL_POINTER;
  if (s.seq_kv > 0 && (!k || !v)) return SMA_ERR_NULL_POINTER;
  if (!aligned(q, 16) || !aligned(o, 16)) return SMA_ERR_MISALIGNED;
  if (s.seq_kv > 0 && (!aligned(k, 16) || !aligned(v, 16))) return SMA_ERR_MISALIGNED;
  if (lse && !aligned(lse, 4)) return SMA_ERR_MISALIGNED;
  if (ws && ws_bytes > 0 && !aligned(ws, 16)) return SMA_ERR_MISALIGNED;
  const size_t kvb = s.seq_kv > 0 ? s.kv_bytes : 0;
  const size_t lb = lse ? s.lse_bytes : 0;
  const size_t wb = ws ? ws_bytes : 0;
  const void* outs[3] = {o, lse, ws};
  const size_t out_n[3] = {s.o_bytes, lb, wb};
  const void* ins[3] = {q, k, v};
  const size_t in_n[3] = {s.q_bytes, kvb, kvb};
  for (int i = 0; i < 3; ++i) {
    for (int j = 0; j < 3; ++j)
      if (overlap(outs[i], out_n[i], ins[j], in_n[j])) return SMA_ERR_ALIASING;
    for (int j = i + 1; j < 3; ++j)
      if (overlap(outs[i], out_n[i], outs[j], out_n[j])) return SMA_ERR_ALIASING;
  }
  return SMA_OK;
}

int validate_all(const void* q, const void* k, const void* v, const void* o, const float* lse,
                 int in_dtype, int o_dtype, size_t batch, size_t heads, size_t seq_q, size_t seq_kv,
                 size_t d, double scale, const void* ws, size_t ws_bytes, Shape* sh,
                 int layout = SMA_LAYOUT_BHSD) {
  int st = check_shape(in_dtype, o_dtype, batch, heads, seq_q, seq_kv, d, scale, sh, layout);
  if (st != SMA_OK) return st;
  if (sh->rows == 0) return SMA_OK;
  st = check_pointers(*sh, q, k, v, o, lse, ws, ws_bytes);
  if (st != SMA_OK) return st;
  const size_t nwg32 = sh->bh * ((sh->seq_q + sma::kF32WsplitQueriesPerWG - 1) / sma::kF32WsplitQueriesPerWG);
  if (nwg32 > kMaxWorkgroups) return SMA_ERR_UNSUPPORTED;
  if ((sh->rows * sh->d / 4 + 255) / 256 > kMaxWorkgroups) return SMA_ERR_UNSUPPORTED;
  return SMA_OK;
}

// Compute units of each device, queried once per device.
constexpr int kMaxDevices = 64;
std::once_flag g_cu_once[kMaxDevices];
int g_cus[kMaxDevices];

int current_device_cus(int* out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return SMA_ERR_HIP;
  std::call_once(g_cu_once[dev], [dev] {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) n = 0;
    g_cus[dev] = n;
  });
  if (g_cus[dev] <= 0) return SMA_ERR_HIP;
  *out = g_cus[dev];
  return SMA_OK;
}

}  // namespace

namespace {

// An optional hard mask: bytes [batches][heads][seq_q][seq_kv], batches 1 or
// B and heads 1 or H (broadcast), nonzero admitting.
struct MaskArg {
  const void* mask = nullptr;
  size_t batches = 0, heads = 0;
};

size_t mask_words(size_t seq_kv) { return (seq_kv + 31) / 32; }

// The column packing of the 16-bit kernel: 32-row blocks and key positions
// (keys rounded up to the 64-key tile).
size_t mask_row_blocks(size_t seq_q) { return (seq_q + 31) / 32; }
size_t mask_key_positions(size_t seq_kv) { return round_up(seq_kv, 64); }
size_t mask_cols_bytes(const Shape& s, const MaskArg& m) {
  return round_up(m.batches * m.heads * mask_row_blocks(s.seq_q) * mask_key_positions(s.seq_kv) * 4,
                  kWsAlign);
}

// Workspace bytes of the mask packed as row words (the fp32 forward kernels
// and every backward kernel); 0 without a mask.
size_t mask_rows_bytes(const Shape& s, const MaskArg& m) {
  if (!m.mask) return 0;
  return round_up(m.batches * m.heads * s.seq_q * mask_words(s.seq_kv) * 4, kWsAlign);
}

// Workspace bytes for the forward's packed mask (0 without a mask): row words
// for the fp32 kernels, column words and tile classes for the 16-bit kernel.
size_t mask_bits_bytes(const Shape& s, const MaskArg& m) {
  if (!m.mask) return 0;
  if (s.in_dtype != SMA_DTYPE_F32)
    return mask_cols_bytes(s, m) +
           round_up(m.batches * m.heads * mask_row_blocks(s.seq_q) * (mask_key_positions(s.seq_kv) / 64) * 4,
                    kWsAlign);
  return mask_rows_bytes(s, m);
}

int check_mask(const Shape& s, const MaskArg& m, const void* o, const float* lse, const void* ws,
               size_t ws_bytes) {
  if (!m.mask) return SMA_OK;
  if ((m.batches != 1 && m.batches != s.batch) || (m.heads != 1 && m.heads != s.heads))
    return SMA_ERR_INVALID_VALUE;
  size_t n;
  if (!mul(m.batches * m.heads, s.seq_q, &n) || !mul(n, s.seq_kv, &n)) return SMA_ERR_INVALID_VALUE;
  if (n > (size_t(1) << 40)) return SMA_ERR_UNSUPPORTED;
  if (s.seq_q * mask_words(s.seq_kv) * 4 > (size_t(1) << 31)) return SMA_ERR_UNSUPPORTED;
  if (overlap(o, s.o_bytes, m.mask, n) || overlap(lse, lse ? s.lse_bytes : 0, m.mask, n) ||
      overlap(ws, ws ? ws_bytes : 0, m.mask, n))
    return SMA_ERR_ALIASING;
  return SMA_OK;
}


// Device scratch of sma_attention_fwd_noalloc: the key-split partials (O and
// log2-unit LSE per split and row). Every automatic plan on a 256-CU device fits
// (at most (2*slots - 2) split-blocks of 256 rows x 129 floats, about 64.5 MiB).
// In host code `scratch` only names the variable: its device address, one per
// GPU, comes from hipGetSymbolAddress (scratch_address below).
constexpr size_t kScratchBytes = size_t(SMA_NOALLOC_SCRATCH_BYTES);
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::once_flag g_scratch_once[kMaxDevices];
void* g_scratch[kMaxDevices];

// The current device's copy of `scratch`, looked up once per device with that
// device current.
int scratch_address(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return SMA_ERR_HIP;
  std::call_once(g_scratch_once[dev], [dev] {
    void* ptr = nullptr;
    g_scratch[dev] = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) == hipSuccess ? ptr : nullptr;
  });
  if (!g_scratch[dev]) return SMA_ERR_HIP;
  *out = g_scratch[dev];
  return SMA_OK;
}

// use_scratch: the workspace is the device's `scratch` (workspace and
// workspace_bytes are ignored); an explicit split that does not fit it is
// SMA_ERR_SCRATCH.
int fwd_core(const void* q, const void* k, const void* v, void* o, float* lse, int in_dtype,
             int o_dtype, size_t batch, size_t heads, size_t seq_q, size_t seq_kv, size_t head_dim,
             double scale, int causal, int layout, const MaskArg& mask, void* workspace,
             size_t workspace_bytes, const sma_plan* plan, void* stream, void* event_before,
             void* event_after, bool use_scratch = false) {
  if (use_scratch) {
    workspace = nullptr;
    workspace_bytes = 0;
  }
  Shape sh;
  int st = validate_all(q, k, v, o, lse, in_dtype, o_dtype, batch, heads, seq_q, seq_kv, head_dim,
                        scale, workspace, workspace_bytes, &sh, layout);
  if (st != SMA_OK) return st;
  const bool masked = mask.mask != nullptr;
  sh.masked = masked;
  if (masked || mask.batches || mask.heads) {
    if (!masked && sh.rows > 0 && seq_kv > 0) return SMA_ERR_NULL_POINTER;
    st = check_mask(sh, mask, o, lse, workspace, workspace_bytes);
    if (st != SMA_OK) return st;
  }
  if (plan) {
    if (plan->nsplit < 1 || plan->nsplit > kMaxSplits) return SMA_ERR_INVALID_VALUE;
    if (plan->kernel != SMA_KERNEL_F32_QBLOCK && plan->kernel != SMA_KERNEL_F32_KSPLIT &&
        plan->kernel != SMA_KERNEL_BF16_QBLOCK)
      return SMA_ERR_INVALID_VALUE;
    if (!kernel_fits_dtype(plan->kernel, in_dtype) || !kernel_fits_head_dim(plan->kernel, sh.d))
      return SMA_ERR_UNSUPPORTED;
    if (plan->kernel == SMA_KERNEL_F32_KSPLIT && (plan->nsplit > 1 || !ksplit_fits(sh)))
      return SMA_ERR_UNSUPPORTED;
  }
  if (sh.rows == 0) return SMA_OK;
  // The packed mask occupies the front of the workspace; a key split uses the rest.
  if (use_scratch) {
    if (mask.mask) return SMA_ERR_INVALID_VALUE;
    st = scratch_address(&workspace);
    if (st != SMA_OK) return st;
    workspace_bytes = kScratchBytes;
  }
  const size_t bits_bytes = mask_bits_bytes(sh, mask);
  if (masked && (!workspace || workspace_bytes < bits_bytes)) return SMA_ERR_INVALID_VALUE;
  void* split_ws = workspace ? static_cast<char*>(workspace) + bits_bytes : nullptr;
  const size_t split_ws_bytes = workspace ? workspace_bytes - bits_bytes : 0;
  int cus = 0;
  st = current_device_cus(&cus);
  if (st != SMA_OK) return st;
  Plan p;
  if (plan) {
    p = plan_for(sh, plan->kernel, (size_t)plan->nsplit, cus);
    if (p.nsplit > 1 && (!split_ws || split_ws_bytes < p.ws_bytes))
      return use_scratch ? SMA_ERR_SCRATCH : SMA_ERR_INVALID_VALUE;
    if (p.nwg > kMaxWorkgroups) return SMA_ERR_UNSUPPORTED;
  } else {
    p = auto_plan(sh, cus);
    if (p.nsplit > 1 && (!split_ws || split_ws_bytes < p.ws_bytes || p.nwg > kMaxWorkgroups))
      p = plan_for(sh, p.kernel, 1, cus);
  }

  sma::FwdArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.bh = (int64_t)sh.bh;
  a.seq_q = (int32_t)seq_q;
  a.seq_kv = (int32_t)seq_kv;
  a.nqb = p.nqb;
  a.nsplit = p.nsplit;
  a.split_len = p.split_len;
  a.c = (float)(std::fabs(scale) * 1.44269504088896340736);  // |scale| * log2(e), one rounding
  a.negate_q = scale < 0.0 ? 1 : 0;
  a.nwg = (uint32_t)p.nwg;
  a.heads = (int64_t)heads;
  if (layout == SMA_LAYOUT_BSHD) {  // element (b, s, h, c) at ((b*S + s)*H + h)*d + c
    a.qs_b = (int64_t)(seq_q * heads * head_dim);
    a.kvs_b = (int64_t)(seq_kv * heads * head_dim);
    a.qs_h = a.kvs_h = (int64_t)head_dim;
    a.qs_s = a.kvs_s = (int64_t)(heads * head_dim);
  } else {  // element (b, h, s, c) at ((b*H + h)*S + s)*d + c
    a.qs_b = (int64_t)(heads * seq_q * head_dim);
    a.kvs_b = (int64_t)(heads * seq_kv * head_dim);
    a.qs_h = (int64_t)(seq_q * head_dim);
    a.kvs_h = (int64_t)(seq_kv * head_dim);
    a.qs_s = a.kvs_s = (int64_t)head_dim;
  }
  const bool o16 = o_dtype != SMA_DTYPE_F32;
  a.o_f16 = o_dtype == SMA_DTYPE_F16 ? 1 : 0;
  if (p.nsplit == 1) {
    if (o16) a.o_bf16 = static_cast<unsigned short*>(o);
    else a.o = static_cast<float*>(o);
    a.lse = lse;
  } else {
    a.part_o = static_cast<float*>(split_ws);
    a.part_lse = reinterpret_cast<float*>(static_cast<char*>(split_ws) + p.part_lse_off);
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool c = causal != 0;
  const int d = (int)head_dim;
  hipError_t e;
  if (masked && seq_kv > 0 && in_dtype != SMA_DTYPE_F32) {
    sma::MaskColArgs mc{};
    mc.mask = static_cast<const unsigned char*>(mask.mask);
    mc.cols = static_cast<uint32_t*>(workspace);
    mc.cls = reinterpret_cast<uint32_t*>(static_cast<char*>(workspace) + mask_cols_bytes(sh, mask));
    mc.slabs = (int64_t)(mask.batches * mask.heads);
    mc.seq_q = (int32_t)seq_q;
    mc.seq_kv = (int32_t)seq_kv;
    mc.nrb = (int32_t)mask_row_blocks(seq_q);
    mc.kpad = (int32_t)mask_key_positions(seq_kv);
    e = sma::launch_mask_pack_cols(mc, s);
    if (e != hipSuccess) return SMA_ERR_HIP;
    a.mask_bits = mc.cols;
    a.mask_words = mc.kpad;
    const int64_t slab = (int64_t)mc.nrb * mc.kpad;
    a.mbits_sh = mask.heads == heads && heads > 1 ? slab : 0;
    a.mbits_sb = mask.batches == batch && batch > 1 ? (int64_t)mask.heads * slab : 0;
    a.mask_cls = mc.cls;
    a.mask_tiles = mc.kpad / 64;
    const int64_t cslab = (int64_t)mc.nrb * a.mask_tiles;
    a.mcls_sh = mask.heads == heads && heads > 1 ? cslab : 0;
    a.mcls_sb = mask.batches == batch && batch > 1 ? (int64_t)mask.heads * cslab : 0;
  } else if (masked && seq_kv > 0) {
    sma::MaskPackArgs mp{};
    mp.mask = static_cast<const unsigned char*>(mask.mask);
    mp.bits = static_cast<uint32_t*>(workspace);
    mp.slabs = (int64_t)(mask.batches * mask.heads);
    mp.seq_q = (int32_t)seq_q;
    mp.seq_kv = (int32_t)seq_kv;
    mp.words = (int32_t)mask_words(seq_kv);
    e = sma::launch_mask_pack(mp, s);
    if (e != hipSuccess) return SMA_ERR_HIP;
    a.mask_bits = mp.bits;
    a.mask_words = mp.words;
    const int64_t slab = (int64_t)seq_q * mp.words;
    a.mbits_sh = mask.heads == heads && heads > 1 ? slab : 0;
    a.mbits_sb = mask.batches == batch && batch > 1 ? (int64_t)mask.heads * slab : 0;
  }
  if (event_before && hipEventRecord(static_cast<hipEvent_t>(event_before), s) != hipSuccess)
    return SMA_ERR_HIP;
  switch (p.kernel) {
    case SMA_KERNEL_F32_KSPLIT: e = sma::launch_fwd_f32_wsplit(a, d, c, s); break;
    case SMA_KERNEL_BF16_QBLOCK: e = sma::launch_fwd_bf16(a, d, c, in_dtype == SMA_DTYPE_F16, s); break;
    default: e = sma::launch_fwd_f32(a, d, c, s); break;
  }
  if (e != hipSuccess) return SMA_ERR_HIP;
  if (event_after && hipEventRecord(static_cast<hipEvent_t>(event_after), s) != hipSuccess)
    return SMA_ERR_HIP;
  if (p.nsplit > 1) {
    sma::CombineArgs ca{};
    ca.part_o = a.part_o;
    ca.part_lse = a.part_lse;
    if (o16) ca.o_bf16 = static_cast<unsigned short*>(o);
    else ca.o = static_cast<float*>(o);
    ca.o_f16 = a.o_f16;
    ca.lse = lse;
    ca.rows = (int64_t)sh.rows;
    ca.nsplit = p.nsplit;
    ca.seq_q = (int32_t)seq_q;
    ca.heads = a.heads;
    ca.os_b = a.qs_b;
    ca.os_h = a.qs_h;
    ca.os_s = a.qs_s;
    e = sma::launch_combine(ca, d, s);
    if (e != hipSuccess) return SMA_ERR_HIP;
  }
  return SMA_OK;
}

}  // namespace

extern "C" {

int sma_attention_fwd_validate(const void* q, const void* k, const void* v, const void* o,
                               const float* lse, int in_dtype, int o_dtype, size_t batch,
                               size_t heads, size_t seq_q, size_t seq_kv, size_t head_dim,
                               double scale, int causal, const void* workspace,
                               size_t workspace_bytes) {
  (void)causal;
  Shape sh;
  return validate_all(q, k, v, o, lse, in_dtype, o_dtype, batch, heads, seq_q, seq_kv, head_dim,
                      scale, workspace, workspace_bytes, &sh);
}

size_t sma_attention_fwd_workspace_bytes(int in_dtype, size_t batch, size_t heads, size_t seq_q,
                                         size_t seq_kv, size_t head_dim, int causal) {
  sma_plan p;
  if (sma_attention_fwd_plan(in_dtype, batch, heads, seq_q, seq_kv, head_dim, causal,
                             SMA_LAYOUT_BHSD, SMA_KERNEL_AUTO, 0, 0, &p) != SMA_OK)
    return 0;
  return p.workspace_bytes;
}

int sma_attention_fwd_plan(int in_dtype, size_t batch, size_t heads, size_t seq_q, size_t seq_kv,
                           size_t head_dim, int causal, int layout, int kernel, int nsplit,
                           int num_cus, sma_plan* out) {
  (void)causal;
  if (!out) return SMA_ERR_NULL_POINTER;
  Shape sh;
  int st = check_shape(in_dtype, SMA_DTYPE_F32, batch, heads, seq_q, seq_kv, head_dim, 1.0, &sh,
                       layout);
  if (st != SMA_OK) return st;
  if (nsplit < 0 || nsplit > kMaxSplits) return SMA_ERR_INVALID_VALUE;
  if (kernel != SMA_KERNEL_AUTO) {
    if (kernel != SMA_KERNEL_F32_QBLOCK && kernel != SMA_KERNEL_F32_KSPLIT &&
        kernel != SMA_KERNEL_BF16_QBLOCK)
      return SMA_ERR_INVALID_VALUE;
    if (!kernel_fits_dtype(kernel, in_dtype) || !kernel_fits_head_dim(kernel, sh.d))
      return SMA_ERR_UNSUPPORTED;
    if (kernel == SMA_KERNEL_F32_KSPLIT && (nsplit > 1 || !ksplit_fits(sh))) return SMA_ERR_UNSUPPORTED;
  }
  int cus = num_cus;
  if (cus <= 0 && current_device_cus(&cus) != SMA_OK) cus = 256;
  Plan p;
  if (sh.rows > 0)
    p = kernel == SMA_KERNEL_AUTO ? auto_plan(sh, cus) : plan_for(sh, kernel, (size_t)nsplit, cus);
  else
    p.kernel = kernel == SMA_KERNEL_AUTO ? auto_kernel(sh, cus) : kernel;
  out->kernel = p.kernel;
  out->nsplit = p.nsplit;
  out->workgroups = p.nwg;
  out->workspace_bytes = p.ws_bytes;
  return SMA_OK;
}

int sma_attention_fwd_ex(const void* q, const void* k, const void* v, void* o, float* lse,
                         int in_dtype, int o_dtype, size_t batch, size_t heads, size_t seq_q,
                         size_t seq_kv, size_t head_dim, double scale, int causal, int layout,
                         void* workspace, size_t workspace_bytes, const sma_plan* plan,
                         void* stream, void* event_before, void* event_after) {
  return fwd_core(q, k, v, o, lse, in_dtype, o_dtype, batch, heads, seq_q, seq_kv, head_dim, scale,
                  causal, layout, MaskArg{}, workspace, workspace_bytes, plan, stream, event_before,
                  event_after);
}

int sma_attention_fwd_masked(const void* q, const void* k, const void* v, void* o, float* lse,
                             const void* mask, size_t mask_batches, size_t mask_heads, int in_dtype,
                             int o_dtype, size_t batch, size_t heads, size_t seq_q, size_t seq_kv,
                             size_t head_dim, double scale, int causal, int layout, void* workspace,
                             size_t workspace_bytes, const sma_plan* plan, void* stream,
                             void* event_before, void* event_after) {
  MaskArg m;
  m.mask = mask;
  m.batches = mask_batches;
  m.heads = mask_heads;
  return fwd_core(q, k, v, o, lse, in_dtype, o_dtype, batch, heads, seq_q, seq_kv, head_dim, scale,
                  causal, layout, m, workspace, workspace_bytes, plan, stream, event_before,
                  event_after);
}

size_t sma_attention_fwd_masked_workspace_bytes(int in_dtype, size_t batch, size_t heads,
                                                size_t seq_q, size_t seq_kv, size_t head_dim,
                                                int causal, int layout, size_t mask_batches,
                                                size_t mask_heads) {
  Shape sh;
  if (check_shape(in_dtype, SMA_DTYPE_F32, batch, heads, seq_q, seq_kv, head_dim, 1.0, &sh,
                  layout) != SMA_OK)
    return 0;
  MaskArg m;
  m.mask = &sh;  // any non-null address: only the sizes matter here
  m.batches = mask_batches;
  m.heads = mask_heads;
  if ((mask_batches != 1 && mask_batches != batch) || (mask_heads != 1 && mask_heads != heads)) return 0;
  // The packed mask, then what the library's key split needs on the current device (the
  // plan of a masked call, whose geometry can differ from the unmasked one).
  (void)causal;
  sh.masked = true;
  int cus = 0;
  if (current_device_cus(&cus) != SMA_OK) cus = 256;
  const size_t split = sh.rows > 0 ? auto_plan(sh, cus).ws_bytes : 0;
  return mask_bits_bytes(sh, m) + split;
}

int sma_attention_fwd_timed(const void* q, const void* k, const void* v, void* o, float* lse,
                            int in_dtype, int o_dtype, size_t batch, size_t heads, size_t seq_q,
                            size_t seq_kv, size_t head_dim, double scale, int causal,
                            void* workspace, size_t workspace_bytes, void* stream,
                            void* event_before, void* event_after) {
  return sma_attention_fwd_ex(q, k, v, o, lse, in_dtype, o_dtype, batch, heads, seq_q, seq_kv,
                              head_dim, scale, causal, SMA_LAYOUT_BHSD, workspace, workspace_bytes,
                              nullptr, stream, event_before, event_after);
}

int sma_attention_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                      int in_dtype, int o_dtype, size_t batch, size_t heads, size_t seq_q,
                      size_t seq_kv, size_t head_dim, double scale, int causal, void* workspace,
                      size_t workspace_bytes, void* stream) {
  return sma_attention_fwd_ex(q, k, v, o, lse, in_dtype, o_dtype, batch, heads, seq_q, seq_kv,
                              head_dim, scale, causal, SMA_LAYOUT_BHSD, workspace, workspace_bytes,
                              nullptr, stream, nullptr, nullptr);
}

int sma_attention_fwd_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                              int in_dtype, int o_dtype, size_t batch, size_t heads, size_t seq_q,
                              size_t seq_kv, size_t head_dim, double scale, int causal, int layout,
                              const sma_plan* plan, void* stream) {
  return fwd_core(q, k, v, o, lse, in_dtype, o_dtype, batch, heads, seq_q, seq_kv, head_dim, scale,
                  causal, layout, MaskArg{}, nullptr, 0, plan, stream, nullptr, nullptr, true);
}

int sma_attention_fwd_layout(const void* q, const void* k, const void* v, void* o, float* lse,
                             int in_dtype, int o_dtype, size_t batch, size_t heads, size_t seq_q,
                             size_t seq_kv, size_t head_dim, double scale, int causal, int layout,
                             void* workspace, size_t workspace_bytes, void* stream) {
  return sma_attention_fwd_ex(q, k, v, o, lse, in_dtype, o_dtype, batch, heads, seq_q, seq_kv,
                              head_dim, scale, causal, layout, workspace, workspace_bytes, nullptr,
                              stream, nullptr, nullptr);
}

// ---------------------------------------------------------------- backward

}  // extern "C"

namespace {

struct BwdShape {
  Shape s;
  size_t nqb, nkb, ws_bytes;
  size_t meta_bytes;     // workspace bytes of the per-block lse2/D (the bf16 dO copy follows)
  size_t q32, kv32;      // bytes of one fp32 [B,H,Sq,d] / [B,H,Skv,d] tensor (o, dout, gradients)
};

// Pointer-independent checks of the backward. Fills b on success.
int check_bwd_shape(int in_dtype, size_t batch, size_t heads, size_t seq_q, size_t seq_kv,
                    size_t d, double scale, BwdShape* b, int layout = SMA_LAYOUT_BHSD) {
  int st = check_shape(in_dtype, SMA_DTYPE_F32, batch, heads, seq_q, seq_kv, d, scale, &b->s, layout);
  if (st != SMA_OK) return st;
  // fp32, bf16 or fp16 Q, K, V; head dims 32, 64 and 128, and 256 with 16-bit inputs.
  if (d != 32 && d != 64 && d != 128 && !(d == 256 && in_dtype != SMA_DTYPE_F32)) return SMA_ERR_UNSUPPORTED;
  // The kernels address one (batch, head) through 32-bit buffer offsets: rows of
  // row_elems elements (heads*d under [B,S,H,d]), with a block of slack.
  const size_t blk = sma::kBwdRowsPerBlock;
  const size_t re = b->s.row_elems;
  if ((seq_q + blk) * re * 4 > (size_t(1) << 31) || (seq_kv + blk) * re * 4 > (size_t(1) << 31))
    return SMA_ERR_UNSUPPORTED;
  b->nqb = (seq_q + blk - 1) / blk;
  b->nkb = (seq_kv + blk - 1) / blk;
  size_t nq, nkv;
  if (!mul(b->s.rows, d, &nq) || !mul(nq, 4, &b->q32) || !mul(b->s.bh, seq_kv, &nkv) ||
      !mul(nkv, d, &nkv) || !mul(nkv, 4, &b->kv32))
    return SMA_ERR_INVALID_VALUE;
  size_t blocks;
  if (!mul(b->s.bh, b->nqb, &blocks) || !mul(blocks, sma::kBwdMetaFloats * sizeof(float), &b->ws_bytes))
    return SMA_ERR_INVALID_VALUE;
  b->ws_bytes = round_up(b->ws_bytes, kWsAlign);
  b->meta_bytes = b->ws_bytes;
  if (in_dtype != SMA_DTYPE_F32) b->ws_bytes += round_up(b->q32 / 2, kWsAlign);  // dO in 16 bits
  if (b->s.bh * b->nqb > kMaxWorkgroups || b->s.bh * b->nkb > kMaxWorkgroups) return SMA_ERR_UNSUPPORTED;
  return SMA_OK;
}

int check_bwd_pointers(const BwdShape& b, const void* q, const void* k, const void* v,
                       const void* o, const float* lse, const void* dout, const float* dq,
                       const float* dk, const float* dv, const void* ws, size_t ws_bytes) {
  const Shape& s = b.s;
  const bool has_q = s.rows > 0, has_kv = s.bh * s.seq_kv > 0;
  if (has_q && (!q || !o || !lse || !dout || !dq)) return SMA_ERR_NULL_POINTER;
  if (has_kv && (!k || !v || !dk || !dv)) return SMA_ERR_NULL_POINTER;
  if (b.ws_bytes > 0 && (!ws || ws_bytes < b.ws_bytes)) return SMA_ERR_INVALID_VALUE;
  const void* t16[] = {q, o, dout, dq, k, v, dk, dv, ws};
  for (const void* p : t16)
    if (p && !aligned(p, 16)) return SMA_ERR_MISALIGNED;
  if (lse && !aligned(lse, 4)) return SMA_ERR_MISALIGNED;
  // Q, K, V in the input type; O, dO and the gradients in fp32.
  const size_t qb = has_q ? s.q_bytes : 0, kvb = has_kv ? s.kv_bytes : 0;
  const size_t q32 = has_q ? b.q32 : 0, kv32 = has_kv ? b.kv32 : 0;
  const size_t lb = has_q ? s.lse_bytes : 0, wb = b.ws_bytes > 0 ? b.ws_bytes : 0;
  const void* outs[4] = {dq, dk, dv, ws};
  const size_t out_n[4] = {q32, kv32, kv32, wb};
  const void* ins[6] = {q, k, v, o, lse, dout};
  const size_t in_n[6] = {qb, kvb, kvb, q32, lb, q32};
  for (int i = 0; i < 4; ++i) {
    for (int j = 0; j < 6; ++j)
      if (overlap(outs[i], out_n[i], ins[j], in_n[j])) return SMA_ERR_ALIASING;
    for (int j = i + 1; j < 4; ++j)
      if (overlap(outs[i], out_n[i], outs[j], out_n[j])) return SMA_ERR_ALIASING;
  }
  return SMA_OK;
}

}  // namespace

extern "C" {

size_t sma_attention_bwd_workspace_bytes(int in_dtype, size_t batch, size_t heads, size_t seq_q,
                                         size_t seq_kv, size_t head_dim, int causal) {
  (void)causal;
  BwdShape b;
  if (check_bwd_shape(in_dtype, batch, heads, seq_q, seq_kv, head_dim, 1.0, &b) != SMA_OK) return 0;
  return b.ws_bytes;
}

}  // extern "C"

namespace {

// A hard mask of the backward: sizes, the packed bits appended to the workspace (b->ws_bytes
// grows by their size, *bits_at is where they start), and no overlap with an output.
int check_bwd_mask(BwdShape* b, const MaskArg& m, const float* dq, const float* dk,
                   const float* dv, const void* ws, size_t* bits_at) {
  const Shape& s = b->s;
  if ((m.batches != 1 && m.batches != s.batch) || (m.heads != 1 && m.heads != s.heads))
    return SMA_ERR_INVALID_VALUE;
  size_t n;
  if (!mul(m.batches * m.heads, s.seq_q, &n) || !mul(n, s.seq_kv, &n)) return SMA_ERR_INVALID_VALUE;
  if (n > (size_t(1) << 40)) return SMA_ERR_UNSUPPORTED;
  if (s.seq_q * mask_words(s.seq_kv) * 4 > (size_t(1) << 31)) return SMA_ERR_UNSUPPORTED;
  *bits_at = b->ws_bytes;
  b->ws_bytes += mask_rows_bytes(s, m);
  if (overlap(dq, s.rows ? b->q32 : 0, m.mask, n) || overlap(dk, b->kv32, m.mask, n) ||
      overlap(dv, b->kv32, m.mask, n) || overlap(ws, ws ? b->ws_bytes : 0, m.mask, n))
    return SMA_ERR_ALIASING;
  return SMA_OK;
}

int bwd_core(const void* q, const void* k, const void* v, const void* o, const float* lse,
             const void* dout, float* dq, float* dk, float* dv, int in_dtype, size_t batch,
             size_t heads, size_t seq_q, size_t seq_kv, size_t head_dim, double scale, int causal,
             int layout, const MaskArg& mask, void* workspace, size_t workspace_bytes, void* stream,
             void* event_after_pre, void* event_after_dkdv) {
  BwdShape b;
  int st = check_bwd_shape(in_dtype, batch, heads, seq_q, seq_kv, head_dim, scale, &b, layout);
  if (st != SMA_OK) return st;
  const bool masked = mask.mask != nullptr;
  size_t bits_at = 0;
  if (masked || mask.batches || mask.heads) {
    if (!masked && b.s.rows > 0 && seq_kv > 0) return SMA_ERR_NULL_POINTER;
    if (masked) {
      st = check_bwd_mask(&b, mask, dq, dk, dv, workspace, &bits_at);
      if (st != SMA_OK) return st;
    }
  }
  st = check_bwd_pointers(b, q, k, v, o, lse, dout, dq, dk, dv, workspace, workspace_bytes);
  if (st != SMA_OK) return st;
  if (b.s.rows == 0 && b.s.bh * seq_kv == 0) return SMA_OK;
  sma::BwdArgs a{};
  a.q = static_cast<const float*>(q);
  a.k = static_cast<const float*>(k);
  a.v = static_cast<const float*>(v);
  a.o = static_cast<const float*>(o);
  a.dout = static_cast<const float*>(dout);
  a.lse = lse;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.meta = static_cast<float*>(workspace);
  if (in_dtype != SMA_DTYPE_F32) {
    a.in_f16 = in_dtype == SMA_DTYPE_F16 ? 1 : 0;
    a.q16 = static_cast<const unsigned short*>(q);
    a.k16 = static_cast<const unsigned short*>(k);
    a.v16 = static_cast<const unsigned short*>(v);
    a.dout16 = reinterpret_cast<unsigned short*>(static_cast<unsigned char*>(workspace) + b.meta_bytes);
  }
  a.bh = (int64_t)b.s.bh;
  a.seq_q = (int32_t)seq_q;
  a.seq_kv = (int32_t)seq_kv;
  a.nqb = (int32_t)b.nqb;
  a.nkb = (int32_t)b.nkb;
  a.c = (float)(scale * 1.44269504088896340736);  // scale * log2(e), one rounding
  a.scale = (float)scale;
  a.heads = (int64_t)heads;
  if (layout == SMA_LAYOUT_BSHD) {  // element (b, s, h, c) at ((b*S + s)*H + h)*d + c
    a.qs_b = (int64_t)(seq_q * heads * head_dim);
    a.kvs_b = (int64_t)(seq_kv * heads * head_dim);
    a.qs_h = a.kvs_h = (int64_t)head_dim;
    a.qs_s = a.kvs_s = (int64_t)(heads * head_dim);
  } else {  // element (b, h, s, c) at ((b*H + h)*S + s)*d + c
    a.qs_b = (int64_t)(heads * seq_q * head_dim);
    a.kvs_b = (int64_t)(heads * seq_kv * head_dim);
    a.qs_h = (int64_t)(seq_q * head_dim);
    a.kvs_h = (int64_t)(seq_kv * head_dim);
    a.qs_s = a.kvs_s = (int64_t)head_dim;
  }
  hipStream_t hs = static_cast<hipStream_t>(stream);
  if (masked && seq_kv > 0 && seq_q > 0) {
    sma::MaskPackArgs mp{};
    mp.mask = static_cast<const unsigned char*>(mask.mask);
    mp.bits = reinterpret_cast<uint32_t*>(static_cast<unsigned char*>(workspace) + bits_at);
    mp.slabs = (int64_t)(mask.batches * mask.heads);
    mp.seq_q = (int32_t)seq_q;
    mp.seq_kv = (int32_t)seq_kv;
    mp.words = (int32_t)mask_words(seq_kv);
    if (sma::launch_mask_pack(mp, hs) != hipSuccess) return SMA_ERR_HIP;
    a.mask_bits = mp.bits;
    a.mask_words = mp.words;
    const int64_t slab = (int64_t)seq_q * mp.words;
    a.mbits_sh = mask.heads == heads && heads > 1 ? slab : 0;
    a.mbits_sb = mask.batches == batch && batch > 1 ? (int64_t)mask.heads * slab : 0;
  }
  const auto launch = in_dtype != SMA_DTYPE_F32 ? sma::launch_bwd_bf16 : sma::launch_bwd_f32;
  hipError_t e = launch(a, (int)head_dim, causal != 0, hs, static_cast<hipEvent_t>(event_after_pre),
                        static_cast<hipEvent_t>(event_after_dkdv));
  return e == hipSuccess ? SMA_OK : SMA_ERR_HIP;
}

}  // namespace

extern "C" {

int sma_attention_bwd_timed(const void* q, const void* k, const void* v, const void* o,
                            const float* lse, const void* dout, float* dq, float* dk, float* dv,
                            int in_dtype, size_t batch, size_t heads, size_t seq_q, size_t seq_kv,
                            size_t head_dim, double scale, int causal, void* workspace,
                            size_t workspace_bytes, void* stream, void* event_after_pre,
                            void* event_after_dkdv) {
  return bwd_core(q, k, v, o, lse, dout, dq, dk, dv, in_dtype, batch, heads, seq_q, seq_kv,
                  head_dim, scale, causal, SMA_LAYOUT_BHSD, MaskArg(), workspace, workspace_bytes,
                  stream, event_after_pre, event_after_dkdv);
}

int sma_attention_bwd(const void* q, const void* k, const void* v, const void* o,
                      const float* lse, const void* dout, float* dq, float* dk, float* dv,
                      int in_dtype, size_t batch, size_t heads, size_t seq_q, size_t seq_kv,
                      size_t head_dim, double scale, int causal, void* workspace,
                      size_t workspace_bytes, void* stream) {
  return bwd_core(q, k, v, o, lse, dout, dq, dk, dv, in_dtype, batch, heads, seq_q, seq_kv,
                  head_dim, scale, causal, SMA_LAYOUT_BHSD, MaskArg(), workspace, workspace_bytes,
                  stream, nullptr, nullptr);
}

int sma_attention_bwd_layout(const void* q, const void* k, const void* v, const void* o,
                             const float* lse, const void* dout, float* dq, float* dk, float* dv,
                             int in_dtype, size_t batch, size_t heads, size_t seq_q,
                             size_t seq_kv, size_t head_dim, double scale, int causal, int layout,
                             void* workspace, size_t workspace_bytes, void* stream) {
  return bwd_core(q, k, v, o, lse, dout, dq, dk, dv, in_dtype, batch, heads, seq_q, seq_kv,
                  head_dim, scale, causal, layout, MaskArg(), workspace, workspace_bytes, stream,
                  nullptr, nullptr);
}

int sma_attention_bwd_masked(const void* q, const void* k, const void* v, const void* o,
                             const float* lse, const void* dout, float* dq, float* dk, float* dv,
                             const void* mask, size_t mask_batches, size_t mask_heads,
                             int in_dtype, size_t batch, size_t heads, size_t seq_q,
                             size_t seq_kv, size_t head_dim, double scale, int causal, int layout,
                             void* workspace, size_t workspace_bytes, void* stream) {
  MaskArg m;
  m.mask = mask;
  m.batches = mask_batches;
  m.heads = mask_heads;
  return bwd_core(q, k, v, o, lse, dout, dq, dk, dv, in_dtype, batch, heads, seq_q, seq_kv,
                  head_dim, scale, causal, layout, m, workspace, workspace_bytes, stream, nullptr,
                  nullptr);
}

size_t sma_attention_bwd_masked_workspace_bytes(int in_dtype, size_t batch, size_t heads,
                                                size_t seq_q, size_t seq_kv, size_t head_dim,
                                                int causal, int layout, size_t mask_batches,
                                                size_t mask_heads) {
  (void)causal;
  BwdShape b;
  if (check_bwd_shape(in_dtype, batch, heads, seq_q, seq_kv, head_dim, 1.0, &b, layout) != SMA_OK)
    return 0;
  if ((mask_batches != 1 && mask_batches != batch) || (mask_heads != 1 && mask_heads != heads)) return 0;
  MaskArg m;
  m.mask = &b;  // any non-null address: only the sizes matter here
  m.batches = mask_batches;
  m.heads = mask_heads;
  return b.ws_bytes + mask_rows_bytes(b.s, m);
}

// ---------------------------------------------------------------- row primitives

}  // extern "C"

namespace {

constexpr size_t kMaxRowCols = (size_t(1) << 31) - 1;  // int32 column math in the kernels
constexpr size_t kMaxRows = (size_t(1) << 31) - 1;     // one workgroup (or a quarter) per row

// Checks shared by the row primitives. out_elems: floats written (rows*cols,
// or rows for the log-sum-exp); out may equal in but not overlap it otherwise.
int check_rows(const float* in, const float* mask, const float* out, bool use_mask, size_t rows,
               size_t cols, size_t out_elems, size_t* in_bytes) {
  size_t n, nb, ob;
  if (!mul(rows, cols, &n) || !mul(n, sizeof(float), &nb) || !mul(out_elems, sizeof(float), &ob))
    return SMA_ERR_INVALID_VALUE;
  if (cols > kMaxRowCols || rows > kMaxRows) return SMA_ERR_UNSUPPORTED;
  if (out_elems > 0 && !out) return SMA_ERR_NULL_POINTER;
  if (n > 0 && (!in || (use_mask && !mask))) return SMA_ERR_NULL_POINTER;
  if ((in && !aligned(in, 4)) || (out && !aligned(out, 4)) || (use_mask && mask && !aligned(mask, 4)))
    return SMA_ERR_MISALIGNED;
  const bool same = (const void*)in == (const void*)out && ob == nb;
  if (!same && overlap(in, nb, out, ob)) return SMA_ERR_ALIASING;
  if (use_mask && overlap(mask, nb, out, ob)) return SMA_ERR_ALIASING;
  *in_bytes = nb;
  return SMA_OK;
}

int launch_row_op(int mode, const float* in, const float* mask, float* out, size_t rows, size_t cols,
                  size_t rows_per_matrix, int causal, double scale, void* stream) {
  sma::RowArgs a{};
  a.in = in;
  a.mask = mask;
  a.out = out;
  a.rows = (int64_t)rows;
  a.cols = (int32_t)cols;
  a.rows_per_matrix = (int32_t)(rows_per_matrix > 0 ? rows_per_matrix : 1);
  a.causal = causal ? 1 : 0;
  a.c = (float)(scale * 1.44269504088896340736);  // scale * log2(e), one rounding
  const bool vec4 = cols % 4 == 0 && aligned(in, 16) && aligned(out, 16) &&
                    (mode != sma::kRowMasked || aligned(mask, 16)) && mode != sma::kRowLse;
  const bool vec4_lse = cols % 4 == 0 && aligned(in, 16);
  const sma::RowPlan plan = sma::plan_rows((int64_t)cols, mode == sma::kRowLse ? vec4_lse : vec4);
  const hipError_t e = sma::launch_rows(mode, a, plan, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? SMA_OK : SMA_ERR_HIP;
}

}  // namespace

extern "C" {

int sma_softmax_rows(const float* in, float* out, size_t rows, size_t cols, void* stream) {
  size_t nb;
  int st = check_rows(in, nullptr, out, false, rows, cols, rows * cols, &nb);
  if (st != SMA_OK || rows == 0 || cols == 0) return st;
  return launch_row_op(sma::kRowSoftmax, in, nullptr, out, rows, cols, 0, 0, 1.0, stream);
}

int sma_logsumexp_rows(const float* in, float* out, size_t rows, size_t cols, void* stream) {
  size_t nb;
  int st = check_rows(in, nullptr, out, false, rows, cols, rows, &nb);
  if (st != SMA_OK || rows == 0) return st;
  return launch_row_op(sma::kRowLse, in, nullptr, out, rows, cols, 0, 0, 1.0, stream);
}

int sma_masked_softmax_rows(const float* in, const float* mask, float* out, size_t rows, size_t cols,
                            void* stream) {
  size_t nb;
  int st = check_rows(in, mask, out, true, rows, cols, rows * cols, &nb);
  if (st != SMA_OK || rows == 0 || cols == 0) return st;
  return launch_row_op(sma::kRowMasked, in, mask, out, rows, cols, 0, 0, 1.0, stream);
}

int sma_scaled_causal_softmax(const float* in, float* out, size_t batch, size_t rows, size_t cols,
                              double scale, int causal, void* stream) {
  if (!std::isfinite(scale)) return SMA_ERR_INVALID_VALUE;
  size_t all_rows;
  if (!mul(batch, rows, &all_rows)) return SMA_ERR_INVALID_VALUE;
  size_t nb;
  int st = check_rows(in, nullptr, out, false, all_rows, cols, all_rows * cols, &nb);
  if (st != SMA_OK || all_rows == 0 || cols == 0) return st;
  return launch_row_op(sma::kRowScaled, in, nullptr, out, all_rows, cols, rows, causal, scale, stream);
}

int sma_softmax_rows_backward(const float* y, const float* dy, float* dx, size_t rows, size_t cols,
                              double scale, void* stream) {
  if (!std::isfinite(scale)) return SMA_ERR_INVALID_VALUE;
  size_t n, nb;
  if (!mul(rows, cols, &n) || !mul(n, sizeof(float), &nb)) return SMA_ERR_INVALID_VALUE;
  if (cols > kMaxRowCols || rows > kMaxRows) return SMA_ERR_UNSUPPORTED;
  if (n == 0) return SMA_OK;
  if (!y || !dy || !dx) return SMA_ERR_NULL_POINTER;
  if (!aligned(y, 4) || !aligned(dy, 4) || !aligned(dx, 4)) return SMA_ERR_MISALIGNED;
  // dx may be y or dy itself (in place), but may not overlap either otherwise.
  if (((const void*)dx != (const void*)y && overlap(y, nb, dx, nb)) ||
      ((const void*)dx != (const void*)dy && overlap(dy, nb, dx, nb)))
    return SMA_ERR_ALIASING;
  sma::RowBwdArgs a{};
  a.y = y;
  a.dy = dy;
  a.dx = dx;
  a.rows = (int64_t)rows;
  a.cols = (int32_t)cols;
  a.scale = (float)scale;
  const bool vec4 = cols % 4 == 0 && aligned(y, 16) && aligned(dy, 16) && aligned(dx, 16);
  const sma::RowPlan plan = sma::plan_rows((int64_t)cols, vec4);
  return sma::launch_rows_bwd(a, plan, static_cast<hipStream_t>(stream)) == hipSuccess ? SMA_OK
                                                                                       : SMA_ERR_HIP;
}

const char* sma_status_string(int status) {
  switch (status) {
    case SMA_OK: return "SMA_OK: success";
    case SMA_ERR_NULL_POINTER: return "SMA_ERR_NULL_POINTER: a required pointer is NULL";
    case SMA_ERR_INVALID_VALUE: return "SMA_ERR_INVALID_VALUE: invalid size, dtype code or scale";
    case SMA_ERR_UNSUPPORTED: return "SMA_ERR_UNSUPPORTED: valid request that the kernels do not implement";
    case SMA_ERR_MISALIGNED: return "SMA_ERR_MISALIGNED: q/k/v/o/workspace need 16-byte and lse 4-byte alignment";
    case SMA_ERR_ALIASING: return "SMA_ERR_ALIASING: an output overlaps an input or another output";
    case SMA_ERR_HIP: return "SMA_ERR_HIP: the HIP runtime reported an error";
    case SMA_ERR_SCRATCH:
      return "SMA_ERR_SCRATCH: the plan's key split needs more than the no-allocation entry "
             "point's device scratch (SMA_NOALLOC_SCRATCH_BYTES)";
    default: return "unknown sma status";
  }
}

int sma_abi_version(void) { return SMA_ABI_VERSION; }

}  // extern "C"
