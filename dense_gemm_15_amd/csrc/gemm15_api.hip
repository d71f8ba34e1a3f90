// gemm15_api.hip -- the C ABI: plans, the shape-bucket configuration choice with
// its exact-shape cache, argument checking and launches.
//
// Configuration choice follows the DeepGEMM page (section 2.3: tile parameters
// per size bucket, repeated shapes served from a cache; section 4.3: a
// small-tile path when M or N is small; section 4.2: a configuration must fit
// the shared-memory and register budget and balance the number of blocks
// against per-block resources). Here the budget is gfx950's 160 KB of LDS per
// workgroup and its compute-unit count, and the balance is an explicit cost
// model: rounds of workgroups over the CUs times the work of one round at the
// configuration's relative efficiency.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <tuple>
#include <vector>

#include "../../include/gemm15.h"
#include "kernels.hpp"
#include "splitk.hpp"
#include "softmax.hpp"
#include "attention.hpp"

using namespace g15;

// Scratch held by the library for gemm_run_noalloc, one copy per GPU the library runs
// on, kept until the process ends: kScratchBytes usable from a 256-byte boundary (the
// array is 256 bytes longer, so the usable part starts at its first 256-byte boundary
// whatever alignment the code object gives it). Host code never uses this name as an
// address: the device address comes from hipGetSymbolAddress (scratch_address below).
// The array has external linkage (in the library's namespace): the runtime finds a
// registered device variable by name among the code object's global symbols, and an
// internal-linkage (static) array is a local symbol there.
constexpr int64_t kScratchBytes = int64_t(16) << 20;
namespace g15 {
__device__ __attribute__((used)) __align__(256) unsigned char scratch[kScratchBytes + 256];
}  // namespace g15

// A plan holds host state only: the choice of configuration and the sizes of the
// scratch its runs use, which the caller passes in (gemm_run_ws).
struct gemm_plan {
  int64_t M, N, K;
  int32_t dtype;
  gemm_epilogue epi;
  int device;
  int config;    // primary configuration
  int fallback;  // configuration for pointers without 16-byte alignment (may equal config)
  int nows;      // configuration run when the plan needs a workspace and none is given
                 // (-1: none exists); it needs no workspace itself
  int64_t batch_hint;
  int64_t workspace_bytes;  // scratch of the primary configuration's runs (0: none)
  int split;        // K split of the primary configuration (resident workgroups: K1 kind)
  int b_nk;         // 1: B is given transposed, Bt [N x K] row-major
  int packed;       // bit 0: A rows padded into the workspace; bit 1: B rows
  int64_t lda_p;    // padded row lengths (elements) of the A and B copies
  int64_t ldb_p;
  int64_t pack_b_off;  // byte offset of the B copy in the workspace (the A copy is at 0)
  // Thin edges (products whose M and N end a few rows / columns past a 256
  // boundary): the primary configuration runs the (M - edge_m) x (N - edge_n) block
  // in whole tiles, the few-row kernel `edge_gemv` (split edge_split, its partial
  // sums at edge_ws_off in the workspace) the last edge_m rows, and the few-column
  // kernel the last edge_n columns of the other rows.
  int edge_m, edge_n;
  int edge_gemv, edge_split;
  int64_t edge_ws_off;
};

namespace {

thread_local int t_last_error = GEMM_OK;

struct Registry {
  std::vector<KernelEntry> all;
  Registry() {
    const KernelEntry* p = nullptr;
    int n = simple_entries(&p);
    all.insert(all.end(), p, p + n);
    n = mfma16_entries(&p);
    all.insert(all.end(), p, p + n);
    n = mfma16_dlds_entries(&p);
    all.insert(all.end(), p, p + n);
    n = mfma16_nt_entries(&p);
    all.insert(all.end(), p, p + n);
    n = f32_entries(&p);
    all.insert(all.end(), p, p + n);
    n = f32_dlds_entries(&p);
    all.insert(all.end(), p, p + n);
    n = gemv_entries(&p);
    all.insert(all.end(), p, p + n);
    n = ladder_entries(&p);
    all.insert(all.end(), p, p + n);
    n = mfma16_k1_entries(&p);
    all.insert(all.end(), p, p + n);
    n = mfma16_w_entries(&p);
    all.insert(all.end(), p, p + n);
  }
};

const Registry& registry() {
  static Registry r;
  return r;
}

int elem_bytes(int dt) { return dt == GEMM_F32 ? 4 : 2; }

bool valid_dtype(int dt) { return dt == GEMM_F32 || dt == GEMM_F16 || dt == GEMM_BF16; }

gemm_epilogue norm_epi(const gemm_epilogue* e) {
  gemm_epilogue d{0u, 1.0f, GEMM_F32};
  return e ? *e : d;
}

// Per configuration: the relative sustained throughput of one CU at full occupancy
// (1.0 = m16d 256 x 256 for the 16-bit types, f32d 256 x 256 for fp32), the fixed
// cost of one tile (prologue, epilogue) in rows of K, and the throughput of a lone
// workgroup of an occupancy-2 configuration relative to a pair. First measured on
// MI355X with square 4096 products (whole rounds of tiles), then refitted on sweeps
// of 16-bit products timed on every main tile configuration (66 shapes, M, N, K
// from 96 to 8192: the model's picks within 0.8% of the per-shape best); m16t is
// fastest up to K of about 4096, m16w beyond (its longer prologue and epilogue
// cost about 250 rows of K per tile). The cost model below adds the rounds of
// tiles a shape needs.
struct EffRow {
  const char* name_prefix;
  double eff;
  double fixed = 64.0;
  double lone = 0.63;
};
const EffRow kEff[] = {
    // bf16 / fp16
    {"m16w_bf16_256x256x32_r4", 1.08, 250.0}, {"m16w_f16_256x256x32_r4", 1.08, 250.0},
    {"m16d_bf16_256x256x64_w4x2_a3_b4_r1", 1.00}, {"m16d_f16_256x256x64_w4x2_a3_b4_r1", 1.00},
    {"m16d_bf16_256x256x64_w2x4_a3_b4_r1", 0.99}, {"m16d_f16_256x256x64_w2x4_a3_b4_r1", 0.99},
    {"m16d_bf16_256x256x64_w2x4_a3_b4_r2", 0.96}, {"m16d_f16_256x256x64_w2x4_a3_b4_r2", 0.96},
    {"m16d_bf16_128x256", 0.84}, {"m16d_f16_128x256", 0.84},
    {"m16d_bf16_256x128x64_w2x2_a4_b4_r1", 0.82}, {"m16d_f16_256x128x64_w2x2_a4_b4_r1", 0.82},
    {"m16d_bf16_256x128", 0.80}, {"m16d_f16_256x128", 0.80},
    {"m16d_bf16_256x256x64_w2x2", 0.88}, {"m16d_f16_256x256x64_w2x2", 0.88},
    {"m16d_bf16_128x128x64_w2x2_a3_b4_r1", 0.81}, {"m16d_f16_128x128x64_w2x2_a3_b4_r1", 0.81},
    {"m16d_bf16_128x128x64_w2x2_a3", 0.79}, {"m16d_f16_128x128x64_w2x2_a3", 0.79},
    {"m16d_bf16_128x128x64_w2x2_a4", 0.67}, {"m16d_f16_128x128x64_w2x2_a4", 0.67},
    {"m16d_bf16_64x128", 0.62}, {"m16d_f16_64x128", 0.62},
    {"m16n_bf16_256x256x64_w2x4", 1.05}, {"m16n_f16_256x256x64_w2x4", 1.05},
    {"m16n_bf16_256x256x64_w4x2", 1.01}, {"m16n_f16_256x256x64_w4x2", 1.01},
    {"m16t_bf16_256x256x64_w2x4", 1.03}, {"m16t_f16_256x256x64_w2x4", 1.03},
    {"m16t_bf16_256x256", 0.97}, {"m16t_f16_256x256", 0.97},
    {"m16t_bf16_128x128x64_w2x2_a2_b2", 0.78}, {"m16t_f16_128x128x64_w2x2_a2_b2", 0.78},
    {"m16t_bf16_128x256", 0.91}, {"m16t_f16_128x256", 0.91},
    // the small direct-to-LDS tile: fitted on 66 measured shapes (best of 13 tiles on 28)
    {"m16t_bf16_64x128", 0.68, 16.0}, {"m16t_f16_64x128", 0.68, 16.0},
    {"m16t_bf16_", 0.75}, {"m16t_f16_", 0.75},
    {"m16n_bf16_128x256", 0.92}, {"m16n_f16_128x256", 0.92},
    {"m16n_bf16_256x128", 0.86}, {"m16n_f16_256x128", 0.86},
    {"m16n_bf16_128x128x64_w2x2_a2_b2", 0.86}, {"m16n_f16_128x128x64_w2x2_a2_b2", 0.86},
    {"m16n_bf16_128x128x64_w2x2_a3_b3", 0.85}, {"m16n_f16_128x128x64_w2x2_a3_b3", 0.85},
    {"m16n_bf16_64x128x64_w2x2_a3_b3", 0.70, 16.0, 1.0}, {"m16n_f16_64x128x64_w2x2_a3_b3", 0.70, 16.0, 1.0},
    {"m16n_bf16_64x128", 0.66}, {"m16n_f16_64x128", 0.66},
    {"mfma16_bf16_128x128_w2x2_scalar", 0.10}, {"mfma16_f16_128x128_w2x2_scalar", 0.10},
    {"mfma16_bf16_64x64_w2x2_scalar", 0.08}, {"mfma16_f16_64x64_w2x2_scalar", 0.08},
    // the register-staged kernels, measured against m16d 64 x 128 on products of 8 to
    // 32 tiles (512^3, 1024^3, M or N of 256 with K up to 1024): 1.3-2x its time
    // even with twice its tiles, so they rank below every direct-to-LDS tile
    {"mfma16_bf16_128x128", 0.20}, {"mfma16_f16_128x128", 0.20},
    {"mfma16_bf16_128x64", 0.15}, {"mfma16_f16_128x64", 0.15},
    {"mfma16_bf16_64x64", 0.16}, {"mfma16_f16_64x64", 0.16},
    // fp32 (relative to the fastest fp32 configuration)
    {"f32d_256x256x16_w4x2_a3", 1.00}, {"f32d_128x256x16_w2x4_a4", 0.95},
    {"f32d_128x128x16_w2x2_a3", 0.95}, {"f32d_128x128x16_w2x2_a4", 0.93},
    {"f32d_256x128x16_w4x2_a4", 0.91},
    {"f32_128x128_w2x2_scalar", 0.63}, {"f32_64x64_w2x2_scalar", 0.55},
    {"f32_128x128", 0.91}, {"f32_128x256", 0.88}, {"f32_256x128", 0.86},
    {"f32_64x64", 0.83}, {"f32_256x256", 0.51},
};

// Measured winners for the shapes of the standard workloads on MI355X (256 CUs,
// 160 KB of LDS per workgroup) (DeepGEMM page, section 2.3: tuned parameters per
// shape bucket). Matched exactly on the device, input class (16-bit or fp32),
// M, N, K and batch; the cost model covers every other shape and device. The
// name's "{t}" stands for the 16-bit type of the problem.
struct TunedRow {
  bool f32;
  int64_t M, N, K, batch;
  const char* config;  // an "m16n" or "_nk" configuration answers a transposed B
};
const TunedRow kTuned[] = {
    // 4096^3 and 8192^3: the one-wave-per-SIMD kernel, in alternating graph-replay
    // runs faster than m16t at 4096^3 (bf16 103.6 against 105.3 us with bf16 output,
    // fp16 109.4 against 111.8 with fp16 output, 111.5 against 117.1 with fp32
    // output) and than m16d at 8192^3 (bf16 763 against 828 us, fp16 814 against 889)
    {false, 4096, 4096, 4096, 1, "m16w_{t}_256x256x32_r4"},
    {false, 8192, 8192, 8192, 1, "m16w_{t}_256x256x32_r4"},
    // 2048^3, 1024^3, 512^3: the 64 x 128 direct-to-LDS tile (fp16, fp32 output: 26.9
    // against 27.9 us for m16d 128 x 128, 10.0 against 11.2 and 6.9 against 7.8 us for
    // m16d 64 x 128)
    {false, 2048, 2048, 2048, 1, "m16t_{t}_64x128x64_w2x2_a3_b3"},
    {false, 1024, 1024, 1024, 1, "m16t_{t}_64x128x64_w2x2_a3_b3"},
    {false, 512, 512, 512, 1, "m16t_{t}_64x128x64_w2x2_a3_b3"},
    {false, 8192, 3072, 768, 1, "m16t_{t}_128x128x64_w2x2_a2_b2"},     // encoder FFN, first GEMM
    {false, 8192, 768, 3072, 1, "m16t_{t}_128x256x64_w2x4_a3_b3"},  // encoder FFN, second GEMM
    {false, 512, 512, 64, 96, "m16s_{t}_256x128x64_w4x2"},             // 96 heads of Q K^T
    {false, 4096, 4096, 4096, 1, "m16n_{t}_256x256x64_w2x4_a3_b2"},
    // transposed B at 8192^3: 825 against 838 us for m16n (bf16)
    {false, 8192, 8192, 8192, 1, "m16w_{t}_256x256x32_r5_nk"},
    {false, 2048, 2048, 2048, 1, "m16n_{t}_128x128x64_w2x2_a3_b3"},
    {false, 8192, 3072, 768, 1, "m16n_{t}_128x128x64_w2x2_a2_b2"},
    {false, 8192, 768, 3072, 1, "m16n_{t}_128x256x64_w2x4_a3_b3"},
    {false, 512, 512, 64, 96, "m16s_{t}_128x128x64_w2x2_nk"},  // Q K^T with K as stored
    {false, 512, 64, 512, 96, "m16t_{t}_128x128x64_w2x2_a2_b2"},  // 96 heads of P V
    {false, 512, 64, 512, 96, "m16n_{t}_128x128x64_w2x2_a2_b2"},
    {true, 4096, 4096, 4096, 1, "f32d_256x256x16_w4x2_a3"},
    {true, 8192, 8192, 8192, 1, "f32d_256x256x16_w4x2_a3"},
    {true, 2048, 2048, 2048, 1, "f32d_128x128x16_w2x2_a3"},
    {true, 1024, 1024, 1024, 1, "f32_64x64_w2x2"},
    {true, 512, 512, 512, 1, "f32_64x64_w2x2"},
};

const EffRow* eff_row(const KernelEntry& k) {
  for (const EffRow& r : kEff)
    if (std::strncmp(k.name, r.name_prefix, std::strlen(r.name_prefix)) == 0) return &r;
  return nullptr;
}

double cfg_efficiency(const KernelEntry& k) {
  if (const EffRow* r = eff_row(k)) return r->eff;
  if (k.kind == KIND_SIMPLE) return 0.03;
  return 0.3;  // other tiles: measured well below the configurations above
}

// Fixed cost of one tile, in rows of K.
double cfg_fixed(const KernelEntry& k) {
  const EffRow* r = eff_row(k);
  return r ? r->fixed : 64.0;
}

double cfg_lone(const KernelEntry& k) {
  const EffRow* r = eff_row(k);
  return r ? r->lone : 0.63;
}

// Workgroups one CU can hold for a configuration (LDS-limited; registers allow
// at least as many for every configuration compiled here).
int cfg_occupancy(const KernelEntry& k, const gemm_device_desc& dev) {
  int occ = k.lds_bytes > 0 ? dev.lds_bytes / k.lds_bytes : 8;
  if (occ < 1) occ = 1;
  if (occ > 2) occ = 2;
  return occ;
}

bool cfg_fits(const KernelEntry& k, int dtype, bool vec_a, bool vec_b, const gemm_device_desc& dev,
              int64_t M, int64_t N, int64_t K, int out_dtype, bool b_nk = false) {
  if (k.in_dtype != -1 && k.in_dtype != dtype) return false;
  if ((k.b_nk != 0) != b_nk) return false;
  if (k.buf32) {
    const int64_t lim = int64_t(1) << 31;
    const int64_t es = elem_bytes(dtype), oe = elem_bytes(out_dtype);
    if (M * K * es >= lim || K * N * es >= lim || M * N * oe >= lim) return false;
    // the tiled kernels address row-major B from the current K slice: the offsets of
    // its bk rows (bk row lengths past the slice start) must stay 32-bit as well
    if (k.kind != KIND_GEMV && !b_nk && static_cast<int64_t>(k.bk) * N * es >= lim) return false;
  }
  if (k.vec_a && !vec_a) return false;
  if (k.vec_b && !vec_b) return false;
  if (k.lds_bytes > dev.lds_bytes) return false;
  if (k.kind == KIND_GEMV && (M > k.bm || K > static_cast<int64_t>(k.bk) * 65535)) return false;
  if (k.kind == KIND_K1 && K > k.bk) return false;
  return true;
}

// Split-K factor of a few-row (GEMV kind) configuration: enough workgroups to
// keep every CU streaming B (about four per CU), each with at least 128 rows
// of K, and never more than bk rows per workgroup (its A staging limit).
int gemv_split(const KernelEntry& k, int64_t N, int64_t K, int64_t batch,
               const gemm_device_desc& dev) {
  const int64_t strips = (N + k.bn - 1) / k.bn;
  const int64_t s_min = (K + k.bk - 1) / k.bk;
  int64_t s = (4 * static_cast<int64_t>(dev.cu_count) + strips * batch - 1) / (strips * batch);
  const int64_t s_rows = (K + 127) / 128;
  if (s > s_rows) s = s_rows;
  if (s < s_min) s = s_min;
  if (s < 1) s = 1;
  return static_cast<int>(s);
}

// Resident workgroups of a K1 configuration: every CU full, a multiple of 8 so
// each XCD runs the same number.
int k1_workgroups(const KernelEntry& k, const gemm_device_desc& dev) {
  return (dev.cu_count * cfg_occupancy(k, dev) + 7) / 8 * 8;
}

// fp32 partial sums [split][bm][N].
int64_t gemv_workspace_bytes(const KernelEntry& k, int64_t N, int split) {
  return split <= 1 ? 0 : static_cast<int64_t>(split) * k.bm * N * 4;
}

// Workgroups of one launch (one batch item for the GEMV kind, which loops).
int64_t cfg_workgroups(const KernelEntry& k, int64_t M, int64_t N, int split, int64_t batch) {
  const int64_t tiles = ((M + k.bm - 1) / k.bm) * ((N + k.bn - 1) / k.bn);
  if (k.kind == KIND_K1) return tiles * batch < split ? (tiles * batch + 7) / 8 * 8 : split;
  if (k.kind == KIND_MFMA16 && split > 1) return tiles * split;  // split-K, one batch item
  return k.kind == KIND_GEMV ? tiles * split : tiles * batch;
}

// Throughput of one CU running c < occ workgroups of an occupancy-occ
// configuration, relative to running occ of them (measured: one 128 x 128
// workgroup alone reaches 0.63 of a pair's throughput).
double concurrency_gain(const KernelEntry& k, int c, int occ) {
  return c >= occ ? 1.0 : cfg_lone(k);
}

constexpr double kRoundUs = 3.0;  // fixed latency per round of workgroups, microseconds

// Modelled time (arbitrary units) of a configuration on a problem: the busiest
// CU's tiles, run occ at a time at the configuration's relative efficiency,
// plus a fixed per-tile cost (prologue, epilogue) that keeps tiny-K shapes honest.
double cfg_cost(const KernelEntry& k, int64_t M, int64_t N, int64_t K, int64_t batch,
                const gemm_device_desc& dev) {
  const int64_t tm = (M + k.bm - 1) / k.bm, tn = (N + k.bn - 1) / k.bn;
  const int64_t tiles = tm * tn * batch;
  const int occ = cfg_occupancy(k, dev);
  const int64_t per_cu = (tiles + dev.cu_count - 1) / dev.cu_count;  // busiest CU
  const int64_t kpad = ((K + k.bk - 1) / k.bk) * k.bk;
  const double tile_work = static_cast<double>(k.bm) * k.bn * kpad;
  double t = 0.0;
  int64_t rounds = 0;
  for (int64_t left = per_cu; left > 0; left -= occ) {
    const int c = static_cast<int>(left < occ ? left : occ);
    t += c * tile_work / (cfg_efficiency(k) * concurrency_gain(k, c, occ));
    ++rounds;
  }
  t += static_cast<double>(per_cu) * k.bm * k.bn * cfg_fixed(k);
  // each round of workgroups also pays a fixed latency (launch, first loads, last
  // stores) whatever its tile: ROUND_US in the units above, where one microsecond is
  // about 2.6e6 (16-bit inputs: a 256 x 256 x 4096 tile at efficiency 1.03 takes
  // ~100 us) or 1.6e5 (fp32: 1/16 of the matrix rate)
  const double unit_per_us = k.in_dtype == DT_F32 ? 1.6e5 : 2.6e6;
  t += static_cast<double>(rounds) * kRoundUs * unit_per_us;
  return t;
}

int tuned_config(const gemm_device_desc& dev, int64_t M, int64_t N, int64_t K, int dtype,
                 int64_t batch, bool b_nk) {
  if (dev.cu_count != 256 || dev.lds_bytes < 163840) return -1;
  const auto& all = registry().all;
  for (const TunedRow& r : kTuned) {
    if (r.f32 != (dtype == GEMM_F32) || r.M != M || r.N != N || r.K != K || r.batch != batch)
      continue;
    std::string name(r.config);
    const size_t at = name.find("{t}");
    if (at != std::string::npos) name.replace(at, 3, dtype == GEMM_BF16 ? "bf16" : "f16");
    for (int i = 0; i < static_cast<int>(all.size()); ++i)
      if (name == all[i].name && (all[i].b_nk != 0) == b_nk) return i;
  }
  return -1;
}

// A configuration choice: the primary configuration, the one taken when the
// pointers are not 16-byte aligned, and which operands go through padded copies.
struct Selection {
  int config = -1;
  int fallback = -1;
  int packed = 0;
  int tile = -1;  // best tile configuration that needs no workspace, for aligned pointers
  int edge = 0;   // 1: thin edges split off (see gemm_plan)
};

// x rounded up to whole 16-byte chunks of es-byte elements
int64_t round_up16B(int64_t x, int64_t es) {
  const int64_t q = 16 / es;
  return (x + q - 1) / q * q;
}

bool is_f32d(const KernelEntry& k) { return std::strncmp(k.name, "f32d_", 5) == 0; }

bool is_m16d(const KernelEntry& k) { return std::strncmp(k.name, "m16d_", 5) == 0; }
bool is_m16t(const KernelEntry& k) { return std::strncmp(k.name, "m16t_", 5) == 0; }

// Split-K factor of a tile configuration on a problem with few tiles and a long K
// (at most half the CUs busy, at least 32 K slices each): S slices of K, each a
// multiple of 8 elements (16-byte aligned A columns) and at least 512 deep, with at
// most two workgroups per CU in all. Measured: 256 x 256 x 4096 11.4 us split 8
// against 28.9 us whole, 128 x 128 x 65536 52.7 against 356 us; 512^3 and 1024^3
// (8 and 16 slices) are faster whole (the partial sums and the second kernel cost
// ~3-10 us). Only the m16d kernels, which take any row strides.
int tile_split(const KernelEntry& k, int64_t M, int64_t N, int64_t K, int64_t batch,
               const gemm_device_desc& dev) {
  if (!is_m16d(k) || K < 2048) return 1;
  const int64_t tiles = ((M + k.bm - 1) / k.bm) * ((N + k.bn - 1) / k.bn) * batch;
  if (2 * tiles > dev.cu_count) return 1;
  for (int S = 32; S >= 2; S /= 2)
    if (K % (8 * S) == 0 && K / S >= 512 && tiles * S <= 2 * dev.cu_count) return S;
  return 1;
}

Selection select_config(const gemm_device_desc& dev, int64_t M, int64_t N, int64_t K, int dtype,
                        const gemm_epilogue& epi, int64_t batch, bool aligned16, bool b_nk) {
  const auto& all = registry().all;
  const int es = elem_bytes(dtype);
  const bool vec_a = aligned16 && (K * es) % 16 == 0;
  const bool vec_b = aligned16 && ((b_nk ? K : N) * es) % 16 == 0;
  // best configuration by the cost model on problem (M, N, K) (ld dims kp, np
  // for the fit of 32-bit offsets), among those `use` accepts
  auto best_for = [&](bool va, bool vb, int64_t kp, int64_t np, auto use, double* cost) {
    int best = -1;
    double best_cost = 0;
    for (int i = 0; i < static_cast<int>(all.size()); ++i) {
      const KernelEntry& k = all[i];
      if (k.kind == KIND_GEMV || k.kind == KIND_LADDER || k.kind == KIND_K1 || !use(k)) continue;
      if (!cfg_fits(k, dtype, va, vb, dev, M, np, kp, epi.out_dtype, b_nk)) continue;
      const double c = cfg_cost(k, M, N, K, batch, dev);
      if (best < 0 || c < best_cost * 0.999) {
        best = i;
        best_cost = c;
      }
    }
    if (cost) *cost = best_cost;
    return best;
  };
  auto any = [](const KernelEntry&) { return true; };
  Selection s;
  s.fallback = best_for(false, false, K, N, any, nullptr);
  s.tile = best_for(vec_a, vec_b, K, N, any, nullptr);
  // A few rows (M <= 8): the product is a stream over B, served by the
  // split-K few-row kernel with the fewest rows that covers M (DeepGEMM page,
  // section 4.3: small shapes get their own small-block kernel).
  for (int i = 0; i < static_cast<int>(all.size()) && !b_nk; ++i) {
    const KernelEntry& k = all[i];
    if (k.kind != KIND_GEMV || !cfg_fits(k, dtype, vec_a, vec_b, dev, M, N, K, epi.out_dtype))
      continue;
    if (s.config < 0 || k.bm < all[s.config].bm) s.config = i;
  }
  if (s.config >= 0) return s;
  const int tuned = tuned_config(dev, M, N, K, dtype, batch, b_nk);
  if (tuned >= 0 && cfg_fits(all[tuned], dtype, vec_a, vec_b, dev, M, N, K, epi.out_dtype, b_nk)) {
    s.config = tuned;
    return s;
  }
  // Few tiles and a long K: when even the smallest m16d tile leaves most CUs idle,
  // that configuration runs the product split along K (the cost model does not
  // model the split). A larger tile is never split instead: where the smallest
  // tile already fills the chip, a split of a larger one measured far slower
  // (bf16 4096 x 2048 x 4096: 256 x 256 split 4 ways 143 us, 128 x 128 tiles 66 us).
  if (!b_nk && dtype != GEMM_F32 && vec_a && vec_b) {
    int pick = -1;
    for (int i = 0; i < static_cast<int>(all.size()); ++i) {
      const KernelEntry& k = all[i];
      if (!is_m16d(k) || !cfg_fits(k, dtype, vec_a, vec_b, dev, M, N, K, epi.out_dtype, b_nk))
        continue;
      if (pick < 0 || k.bm * k.bn < all[pick].bm * all[pick].bn) pick = i;
    }
    if (pick >= 0 && tile_split(all[pick], M, N, K, batch, dev) >= 2) {
      s.config = pick;
      return s;
    }
  }
  double cost = 0;
  s.config = best_for(vec_a, vec_b, K, N, any, &cost);
  const bool pa = (K * es) % 16 != 0, pb = ((b_nk ? K : N) * es) % 16 != 0;
  // Products whose M and N end at most 8 rows / columns past a multiple of 256 (4097^3)
  // and whose whole-tile block fills every CU: whole tiles would leave a second round of
  // one-row tiles, each as slow as a full one (bf16 4097^3 on the best tiling: 252 us
  // against 116 us at 4096^3); the 256 x 256 kernel of the input type takes the
  // whole-tile block in full rounds and the few-row and few-column kernels the edges
  // (operands copied into padded rows when theirs are not 16-byte multiples).
  if (!b_nk && aligned16 && K >= 256 && M % 256 <= 8 && N % 256 <= 8 &&
      M % 256 + N % 256 > 0 && (M / 256) * (N / 256) >= dev.cu_count) {
    const std::string main_cfg = dtype == GEMM_F32 ? std::string("f32d_256x256x16_w4x2_a3")
                                 : std::string("m16t_") + (dtype == GEMM_BF16 ? "bf16" : "f16") +
                                       "_256x256x64_w2x4_a3_b2";
    for (size_t i = 0; i < all.size(); ++i)
      if (main_cfg == all[i].name &&
          cfg_fits(all[i], dtype, true, true, dev, M, N, round_up16B(K, es), epi.out_dtype)) {
        s.config = static_cast<int>(i);
        s.packed = (pa ? 1 : 0) | (pb ? 2 : 0);
        s.edge = 1;
        return s;
      }
  }
  // 16-bit rows that are not 16-byte multiples, K within one 64-deep slice and a
  // large C: the streaming kernel's register-load form reads the rows as they are
  // (no padded copies, no workspace) while C of the previous tile leaves.
  if (dtype != GEMM_F32 && aligned16 && (pa || pb) && K <= 64 &&
      static_cast<double>(M) * N >= double(1 << 22)) {
    const std::string want = std::string("m16s_") + (dtype == GEMM_BF16 ? "bf16" : "f16") +
                             "_256x128x64_w4x2" + (b_nk ? "_nk" : "") + "_u";
    for (size_t i = 0; i < all.size(); ++i)
      if (want == all[i].name &&
          cfg_fits(all[i], dtype, vec_a, vec_b, dev, M, N, K, epi.out_dtype, b_nk)) {
        s.config = static_cast<int>(i);
        return s;
      }
  }
  // Other rows that are not 16-byte multiples: rather than a scalar-load kernel,
  // copy the offending operand into zero-padded rows (plan workspace) and run a
  // 16-byte-load kernel, when the product is big enough to repay the copy (always for
  // a transposed B, which has no scalar-load kernel; fp32 from 2^27 multiply-adds,
  // where the copies cost a few percent of the product and f32d runs 1.6-1.8x the
  // scalar-load kernel).
  const double mnk = static_cast<double>(M) * N * K;
  const bool repays = M > 8 && mnk >= (dtype == GEMM_F32 ? double(1 << 27) : double(1 << 20));
  if (aligned16 && (pa || pb) && (b_nk || repays)) {
    double pcost = 0;
    const int pk = best_for(true, true, pa ? round_up16B(K, es) : K,
                            (pb && !b_nk) ? round_up16B(N, es) : N,
                            [&](const KernelEntry& k) {
                              return dtype == GEMM_F32 ? is_f32d(k)
                                                       : (b_nk || is_m16d(k) || is_m16t(k));
                            },
                            &pcost);
    if (pk >= 0 && (s.config < 0 || pcost < cost)) {
      s.config = pk;
      s.packed = (pa ? 1 : 0) | (pb ? 2 : 0);
    }
  }
  return s;
}

struct CacheKey {
  int64_t M, N, K, batch;
  int dtype, flags, out_dtype, aligned, cu, lds, b_nk;
  bool operator<(const CacheKey& o) const {
    return std::tie(M, N, K, batch, dtype, flags, out_dtype, aligned, cu, lds, b_nk) <
           std::tie(o.M, o.N, o.K, o.batch, o.dtype, o.flags, o.out_dtype, o.aligned, o.cu, o.lds,
                    o.b_nk);
  }
};

struct Cache {
  std::mutex mu;
  std::map<CacheKey, Selection> map;
  int64_t hits = 0, misses = 0;
};

Cache& cache() {
  static Cache c;
  return c;
}

int forced_config() {
  const char* s = std::getenv("GEMM15_FORCE_CONFIG");
  if (!s || !*s) return -1;
  const auto& all = registry().all;
  for (int i = 0; i < static_cast<int>(all.size()); ++i)
    if (std::strcmp(all[i].name, s) == 0) return i;
  return -2;
}

// Cached choice for (shape, types, device facts).
Selection choose(const gemm_device_desc& dev, int64_t M, int64_t N, int64_t K, int dtype,
                 const gemm_epilogue& epi, int64_t batch, bool aligned16, bool b_nk) {
  CacheKey key{M, N, K, batch, dtype, static_cast<int>(epi.flags), epi.out_dtype,
               aligned16 ? 1 : 0, dev.cu_count, dev.lds_bytes, b_nk ? 1 : 0};
  Cache& c = cache();
  {
    std::lock_guard<std::mutex> lk(c.mu);
    auto it = c.map.find(key);
    if (it != c.map.end()) {
      ++c.hits;
      return it->second;
    }
  }
  // chosen outside the lock; a thread that raced another one on the same shape finds
  // its entry here and counts a hit, so misses = entries
  const Selection sel = select_config(dev, M, N, K, dtype, epi, batch, aligned16, b_nk);
  std::lock_guard<std::mutex> lk(c.mu);
  const auto ins = c.map.try_emplace(key, sel);
  if (ins.second)
    ++c.misses;
  else
    ++c.hits;
  return ins.first->second;
}

int check_problem(int64_t M, int64_t N, int64_t K, int32_t dtype, const gemm_epilogue& e,
                  int64_t batch) {
  if (M < 1 || N < 1 || K < 1) return GEMM_ERR_SHAPE;
  if (batch < 1) return GEMM_ERR_ARG;
  if (!valid_dtype(dtype) || !valid_dtype(e.out_dtype)) return GEMM_ERR_DTYPE;
  if (e.flags & ~0xFu) return GEMM_ERR_DTYPE;
  if (!std::isfinite(e.scale)) return GEMM_ERR_ARG;
  // element indices are 64-bit; tile ids and batch index must fit the grid
  if (M > (int64_t(1) << 31) || N > (int64_t(1) << 31) || K > (int64_t(1) << 31))
    return GEMM_ERR_SHAPE;
  return GEMM_OK;
}

int device_desc(int dev, gemm_device_desc* out) {
  static std::mutex mu;
  static std::map<int, gemm_device_desc> known;
  std::lock_guard<std::mutex> lk(mu);
  auto it = known.find(dev);
  if (it != known.end()) {
    *out = it->second;
    return GEMM_OK;
  }
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return GEMM_ERR_HIP;
  gemm_device_desc d;
  d.cu_count = prop.multiProcessorCount;
  d.lds_bytes = static_cast<int32_t>(prop.sharedMemPerBlock);
  if (d.lds_bytes <= 0) d.lds_bytes = 65536;
  known[dev] = d;
  *out = d;
  return GEMM_OK;
}

gemm_plan* fail(int code) {
  t_last_error = code;
  return nullptr;
}

bool aligned_to(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// One batch item at a time: copy the unaligned operand(s) into the plan's
// padded buffers, then run the 16-byte-load kernel with the padded row strides.
int run_packed(const gemm_plan* p, int64_t batch, const void* A, int64_t sA, const void* B,
               int64_t sB, const float* bias, const void* resid, int64_t sR, void* C, int64_t sC,
               bool c16, void* ws, hipStream_t s) {
  const KernelEntry& k = registry().all[p->config];
  const int64_t ie = elem_bytes(p->dtype), oe = elem_bytes(p->epi.out_dtype);
  void* const pack_a = ws;
  void* const pack_b = static_cast<char*>(ws) + p->pack_b_off;
  for (int64_t z = 0; z < batch; ++z) {
    const char* Az = static_cast<const char*>(A) + z * sA * ie;
    const char* Bz = static_cast<const char*>(B) + z * sB * ie;
    auto pack = p->dtype == GEMM_F32 ? pack_rows32 : pack_rows16;
    if ((p->packed & 1) && pack(Az, p->M, p->K, pack_a, p->lda_p, s) != hipSuccess)
      return GEMM_ERR_HIP;
    if ((p->packed & 2) && pack(Bz, p->b_nk ? p->N : p->K, p->b_nk ? p->K : p->N, pack_b,
                                p->ldb_p, s) != hipSuccess)
      return GEMM_ERR_HIP;
    LaunchArgs la;
    la.M = p->M;
    la.N = p->N;
    la.K = p->K;
    la.batch = 1;
    la.A = (p->packed & 1) ? pack_a : Az;
    la.sA = 0;
    la.B = (p->packed & 2) ? pack_b : Bz;
    la.sB = 0;
    la.C = static_cast<char*>(C) + z * sC * oe;
    la.sC = 0;
    la.sR = 0;
    la.epi.flags = p->epi.flags;
    la.epi.scale = p->epi.scale;
    la.epi.bias = bias;
    la.epi.resid = (p->epi.flags & GEMM_EPI_RESID) ? static_cast<const char*>(resid) + z * sR * oe
                                                   : nullptr;
    la.epi.out_dtype = p->epi.out_dtype;
    la.workspace = nullptr;
    la.workspace_bytes = 0;
    la.split = k.kind == KIND_K1 ? p->split : 1;  // resident workgroups of a streaming kernel
    la.lda = p->lda_p;
    la.ldb = p->ldb_p;  // padded, or the unpadded row length
    la.ldc = p->N;
    la.c_vec = (c16 && p->N % 8 == 0) ? 1 : 0;
    if (k.launch(la, s) != hipSuccess) return GEMM_ERR_HIP;
  }
  return GEMM_OK;
}

// Run of a plan with thin edges split off: per batch item, the padded copies
// (if any), the whole-tile block on the primary configuration, the last edge_m rows
// on the few-row kernel (partial sums in the workspace) and the last edge_n columns of
// the other rows on the few-column kernel. C, the residual and the bias are addressed
// at the block's origin with C's full row stride.
int run_edges(const gemm_plan* p, int64_t batch, const void* A, int64_t sA, const void* B,
              int64_t sB, const float* bias, const void* resid, int64_t sR, void* C, int64_t sC,
              bool c16, void* ws, hipStream_t s) {
  const auto& all = registry().all;
  const KernelEntry& k = all[p->config];
  const int64_t ie = elem_bytes(p->dtype), oe = elem_bytes(p->epi.out_dtype);
  const int64_t M1 = p->M - p->edge_m, N1 = p->N - p->edge_n;
  void* const pack_a = ws;
  void* const pack_b = static_cast<char*>(ws) + p->pack_b_off;
  auto base = [&](int64_t m_rows, int64_t n_cols, int64_t K, const void* Ap, int64_t lda,
                  const void* Bp, int64_t ldb, void* Cp, const void* Rp, const float* bp) {
    LaunchArgs la{};
    la.M = m_rows;
    la.N = n_cols;
    la.K = K;
    la.batch = 1;
    la.A = Ap;
    la.B = Bp;
    la.C = Cp;
    la.epi.flags = p->epi.flags;
    la.epi.scale = p->epi.scale;
    la.epi.bias = bp;
    la.epi.resid = Rp;
    la.epi.out_dtype = p->epi.out_dtype;
    la.split = 1;
    la.lda = lda;
    la.ldb = ldb;
    la.ldc = p->N;
    la.c_vec = 0;
    return la;
  };
  auto pack = p->dtype == GEMM_F32 ? pack_rows32 : pack_rows16;
  for (int64_t z = 0; z < batch; ++z) {
    const char* Az = static_cast<const char*>(A) + z * sA * ie;
    const char* Bz = static_cast<const char*>(B) + z * sB * ie;
    char* Cz = static_cast<char*>(C) + z * sC * oe;
    const char* Rz = (p->epi.flags & GEMM_EPI_RESID) ? static_cast<const char*>(resid) + z * sR * oe
                                                     : nullptr;
    if ((p->packed & 1) && pack(Az, p->M, p->K, pack_a, p->lda_p, s) != hipSuccess)
      return GEMM_ERR_HIP;
    if ((p->packed & 2) && pack(Bz, p->K, p->N, pack_b, p->ldb_p, s) != hipSuccess)
      return GEMM_ERR_HIP;
    const char* Au = (p->packed & 1) ? static_cast<const char*>(pack_a) : Az;
    const char* Bu = (p->packed & 2) ? static_cast<const char*>(pack_b) : Bz;
    const int64_t lda = p->lda_p, ldb = p->ldb_p;  // K and N when not copied
    LaunchArgs la = base(M1, N1, p->K, Au, lda, Bu, ldb, Cz, Rz, bias);
    la.c_vec = (c16 && p->N % 8 == 0) ? 1 : 0;  // 16-bit C rows 16-byte aligned: staged stores
    if (k.launch(la, s) != hipSuccess) return GEMM_ERR_HIP;
    if (p->edge_m > 0) {
      LaunchArgs lg = base(p->edge_m, p->N, p->K, Au + M1 * lda * ie, lda, Bu, ldb,
                           Cz + M1 * p->N * oe, Rz ? Rz + M1 * p->N * oe : nullptr, bias);
      lg.split = p->edge_split;
      lg.workspace = static_cast<char*>(ws) + p->edge_ws_off;
      lg.workspace_bytes = p->workspace_bytes - p->edge_ws_off;
      if (all[p->edge_gemv].launch(lg, s) != hipSuccess) return GEMM_ERR_HIP;
    }
    if (p->edge_n > 0) {
      LaunchArgs lc = base(M1, p->edge_n, p->K, Au, lda, Bu + N1 * ie, ldb, Cz + N1 * oe,
                           Rz ? Rz + N1 * oe : nullptr, bias ? bias + N1 : nullptr);
      if (launch_gemv_cols(lc, p->dtype, s) != hipSuccess) return GEMM_ERR_HIP;
    }
  }
  return GEMM_OK;
}

// Split-K run of a tile configuration: the S slices of K run as the S items of one
// strided batch (A advanced Kc columns, B Kc rows, K = Kc, C the workspace's fp32
// partial products, no epilogue; A's row stride stays K, and the kernel's K tail
// keeps each item inside its slice), then the reduction kernel adds the partials in
// slice order and applies the epilogue. Batch items run one after the other and
// share the workspace.
int run_split_k(const gemm_plan* p, const KernelEntry& k, int64_t batch, const void* A,
                int64_t sA, const void* B, int64_t sB, const float* bias, const void* resid,
                int64_t sR, void* C, int64_t sC, void* ws, hipStream_t s) {
  const int S = p->split;
  const int64_t kc = p->K / S;
  const int64_t ie = elem_bytes(p->dtype);
  for (int64_t z = 0; z < batch; ++z) {
    LaunchArgs la{};
    la.M = p->M;
    la.N = p->N;
    la.K = kc;
    la.batch = S;
    la.A = static_cast<const char*>(A) + z * sA * ie;
    la.sA = kc;
    la.B = static_cast<const char*>(B) + z * sB * ie;
    la.sB = kc * p->N;
    la.C = ws;
    la.sC = p->M * p->N;
    la.sR = 0;
    la.epi.flags = 0;
    la.epi.scale = 1.f;
    la.epi.bias = nullptr;
    la.epi.resid = nullptr;
    la.epi.out_dtype = DT_F32;
    la.workspace = nullptr;
    la.workspace_bytes = 0;
    la.split = 1;
    la.lda = p->K;
    la.ldb = p->N;
    la.ldc = p->N;
    la.c_vec = 1;
    if (k.launch(la, s) != hipSuccess) return GEMM_ERR_HIP;
    LaunchArgs lr{};
    lr.M = p->M;
    lr.N = p->N;
    lr.K = p->K;
    lr.batch = 1;
    lr.C = C;
    lr.sC = sC;
    lr.sR = sR;
    lr.epi.flags = p->epi.flags;
    lr.epi.scale = p->epi.scale;
    lr.epi.bias = bias;
    lr.epi.resid = resid;
    lr.epi.out_dtype = p->epi.out_dtype;
    lr.workspace = ws;
    lr.workspace_bytes = p->workspace_bytes;
    lr.split = S;
    lr.lda = p->K;
    lr.ldb = p->N;
    lr.ldc = p->N;
    if (launch_splitk_reduce(lr, z, p->M, s) != hipSuccess) return GEMM_ERR_HIP;
  }
  return GEMM_OK;
}

// Device address of the scratch array on `dev` (the current device), looked up once per
// device with hipGetSymbolAddress and rounded up to a 256-byte boundary; nullptr when
// the lookup fails.
void* scratch_address(int dev) {
  static std::mutex mu;
  static std::map<int, void*> addr;
  std::lock_guard<std::mutex> lk(mu);
  auto it = addr.find(dev);
  if (it != addr.end()) return it->second;
  void* p = nullptr;
  if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) {
    (void)hipGetLastError();
    return nullptr;
  }
  const uintptr_t u = (reinterpret_cast<uintptr_t>(p) + 255) & ~uintptr_t(255);
  addr[dev] = reinterpret_cast<void*>(u);
  return addr[dev];
}

// One-line description of a plan (its configuration choice, for logs and tuning).
int describe_plan(const gemm_plan* p, char* buf, size_t len) {
  const auto& all = registry().all;
  const KernelEntry& k = all[p->config];
  char tmp[384];
  const int n = std::snprintf(
      tmp, sizeof(tmp),
      "config=%s id=%d tile=%dx%dx%d threads=%d lds=%d workgroups=%lld split=%d packed=%d "
      "b=%s fallback=%s workspace=%lld nows=%s edge=%d,%d",
      k.name, p->config, k.bm, k.bn, k.bk, k.threads, k.lds_bytes,
      static_cast<long long>(cfg_workgroups(k, p->M, p->N, p->split, p->batch_hint)),
      k.kind == KIND_K1 ? 1 : p->split,  // a K1 plan keeps its resident workgroups there
      p->packed, p->b_nk ? "nk" : "kn", p->fallback >= 0 ? all[p->fallback].name : "none",
      static_cast<long long>(p->workspace_bytes), p->nows >= 0 ? all[p->nows].name : "none",
      p->edge_m, p->edge_n);
  if (buf && len > 0) {
    std::strncpy(buf, tmp, len - 1);
    buf[len - 1] = '\0';
  }
  return n;
}

// GEMM15_POISON set (and not "0"): every run first fills C with NaN (read per call, so a
// test or a debugging session can switch it on at any time).
bool poison_enabled() {
  const char* s = std::getenv("GEMM15_POISON");
  return s && *s && std::strcmp(s, "0") != 0;
}

// GEMM15_LOG set (and not "0"): every plan creation prints its choice to stderr.
bool log_enabled() {
  static const bool on = [] {
    const char* s = std::getenv("GEMM15_LOG");
    return s && *s && std::strcmp(s, "0") != 0;
  }();
  return on;
}

}  // namespace

extern "C" {

gemm_plan* gemm_plan_create_layout(int64_t M, int64_t N, int64_t K, int32_t dtype,
                                   const gemm_epilogue* epi_in, int64_t batch_hint, int32_t config,
                                   int32_t b_layout) {
  const gemm_epilogue epi = norm_epi(epi_in);
  int rc = check_problem(M, N, K, dtype, epi, batch_hint);
  if (rc) return fail(rc);
  if (b_layout != GEMM_B_KN && b_layout != GEMM_B_NK) return fail(GEMM_ERR_ARG);
  const bool b_nk = b_layout == GEMM_B_NK;
  int ndev = 0;
  if (hipGetDeviceCount(&ndev) != hipSuccess || ndev < 1) return fail(GEMM_ERR_NO_DEVICE);
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return fail(GEMM_ERR_HIP);
  gemm_device_desc desc;
  rc = device_desc(dev, &desc);
  if (rc) return fail(rc);

  const auto& all = registry().all;
  Selection sel;
  const int forced = config >= 0 ? config : forced_config();
  if (forced == -2) return fail(GEMM_ERR_CONFIG);
  if (forced >= 0) {
    if (forced >= static_cast<int>(all.size())) return fail(GEMM_ERR_CONFIG);
    const KernelEntry& k = all[forced];
    const int es = elem_bytes(dtype);
    if (!cfg_fits(k, dtype, (K * es) % 16 == 0, ((b_nk ? K : N) * es) % 16 == 0, desc, M, N, K,
                  epi.out_dtype, b_nk))
      return fail(GEMM_ERR_CONFIG);
    sel.config = forced;
    sel.fallback = forced;
    if (k.vec_a || k.vec_b)
      sel.fallback = select_config(desc, M, N, K, dtype, epi, batch_hint, false, b_nk).config;
  } else {
    sel = choose(desc, M, N, K, dtype, epi, batch_hint, true, b_nk);
  }
  const int cfg = sel.config, fb = sel.fallback;
  // a transposed B has no scalar-load kernel: unaligned pointers are an error at run time
  if (cfg < 0 || (fb < 0 && !b_nk)) return fail(GEMM_ERR_CONFIG);

  gemm_plan* p = new (std::nothrow) gemm_plan();
  if (!p) return fail(GEMM_ERR_NOMEM);
  p->M = M;
  p->N = N;
  p->K = K;
  p->dtype = dtype;
  p->epi = epi;
  p->device = dev;
  p->config = cfg;
  p->fallback = fb;
  p->batch_hint = batch_hint;
  p->workspace_bytes = 0;
  p->split = 1;
  p->b_nk = b_nk ? 1 : 0;
  p->packed = sel.packed;
  const int64_t es = elem_bytes(dtype);
  p->lda_p = (sel.packed & 1) ? round_up16B(K, es) : K;
  p->ldb_p = b_nk ? ((sel.packed & 2) ? round_up16B(K, es) : K)
                  : ((sel.packed & 2) ? round_up16B(N, es) : N);
  p->pack_b_off = 0;
  if (sel.packed) {
    const int64_t a_bytes = (sel.packed & 1) ? M * p->lda_p * es : 0;
    const int64_t b_bytes = (sel.packed & 2) ? (b_nk ? N : K) * p->ldb_p * es : 0;
    p->pack_b_off = (a_bytes + 255) / 256 * 256;
    p->workspace_bytes = p->pack_b_off + b_bytes;
  }
  const KernelEntry& k = all[cfg];
  if (k.kind == KIND_K1) p->split = k1_workgroups(k, desc);
  if (k.kind == KIND_MFMA16 && !sel.packed && !b_nk) {
    p->split = tile_split(k, M, N, K, batch_hint, desc);
    if (p->split > 1) p->workspace_bytes = static_cast<int64_t>(p->split) * M * N * 4;
  }
  if (k.kind == KIND_GEMV) {
    p->split = gemv_split(k, N, K, batch_hint, desc);
    p->workspace_bytes = gemv_workspace_bytes(k, N, p->split);
  }
  p->edge_m = p->edge_n = 0;
  p->edge_gemv = -1;
  p->edge_split = 1;
  p->edge_ws_off = 0;
  if (sel.edge) {
    p->edge_m = static_cast<int>(M % 256);
    p->edge_n = static_cast<int>(N % 256);
    if (p->edge_m > 0) {
      for (int i = 0; i < static_cast<int>(all.size()); ++i) {
        const KernelEntry& g = all[i];
        if (g.kind != KIND_GEMV || g.in_dtype != dtype || g.bm < p->edge_m ||
            !cfg_fits(g, dtype, true, true, desc, p->edge_m, N, K, epi.out_dtype))
          continue;
        if (p->edge_gemv < 0 || g.bm < all[p->edge_gemv].bm) p->edge_gemv = i;
      }
      if (p->edge_gemv < 0) {
        delete p;
        return fail(GEMM_ERR_CONFIG);
      }
      const KernelEntry& g = all[p->edge_gemv];
      p->edge_split = gemv_split(g, N, K, 1, desc);
      p->edge_ws_off = (p->workspace_bytes + 255) / 256 * 256;
      p->workspace_bytes = p->edge_ws_off + gemv_workspace_bytes(g, N, p->edge_split);
    }
  }
  // Without a workspace: the same kernel with K unsplit when it can take all of K,
  // otherwise the best plain tile configuration; padded copies give way to the
  // scalar-load configuration (none for a transposed B).
  p->nows = cfg;
  if (sel.edge) {
    // the whole product on the best plain configuration (no edges split off)
    p->nows = sel.packed ? fb : (sel.tile >= 0 ? sel.tile : fb);
  } else if (sel.packed) {
    p->nows = b_nk ? -1 : fb;
  } else if (k.kind == KIND_GEMV && p->split > 1 && K > k.bk) {
    int t = sel.tile;
    if (forced >= 0) t = select_config(desc, M, N, K, dtype, epi, batch_hint, true, b_nk).tile;
    p->nows = t >= 0 ? t : fb;
  }
  if (log_enabled()) {
    char line[512];
    describe_plan(p, line, sizeof(line));
    std::fprintf(stderr, "gemm15: plan M=%lld N=%lld K=%lld dtype=%d flags=%u out=%d batch=%lld: %s\n",
                 static_cast<long long>(M), static_cast<long long>(N), static_cast<long long>(K),
                 dtype, epi.flags, epi.out_dtype, static_cast<long long>(batch_hint), line);
  }
  return p;
}

gemm_plan* gemm_plan_create_ex(int64_t M, int64_t N, int64_t K, int32_t dtype,
                               const gemm_epilogue* epi, int64_t batch_hint, int32_t config) {
  return gemm_plan_create_layout(M, N, K, dtype, epi, batch_hint, config, GEMM_B_KN);
}

gemm_plan* gemm_plan_create(int64_t M, int64_t N, int64_t K, int32_t dtype,
                            const gemm_epilogue* epi) {
  return gemm_plan_create_layout(M, N, K, dtype, epi, 1, -1, GEMM_B_KN);
}

int gemm_softmax_rows(const float* S, int64_t rows, int64_t cols, int64_t ld_s, float scale,
                      void* P, int64_t ld_p, int32_t p_dtype, void* stream) {
  if (rows < 1 || cols < 1 || (rows + 3) / 4 > 0x7fffffff) return GEMM_ERR_SHAPE;
  if (ld_s < cols || ld_p < cols) return GEMM_ERR_ARG;
  if (p_dtype != GEMM_F32 && p_dtype != GEMM_F16 && p_dtype != GEMM_BF16) return GEMM_ERR_DTYPE;
  if (!S || !P) return GEMM_ERR_NULL;
  if (!aligned_to(S, 4) || !aligned_to(P, elem_bytes(p_dtype))) return GEMM_ERR_ALIGN;
  if (!std::isfinite(scale)) return GEMM_ERR_ARG;
  int ndev = 0;
  if (hipGetDeviceCount(&ndev) != hipSuccess || ndev < 1) return GEMM_ERR_NO_DEVICE;
  const int dt = p_dtype == GEMM_F32 ? DT_F32 : p_dtype == GEMM_BF16 ? DT_BF16 : DT_F16;
  const hipError_t err = launch_softmax_rows(S, rows, cols, ld_s, scale, P, ld_p, dt,
                                             static_cast<hipStream_t>(stream));
  return err == hipSuccess ? GEMM_OK : GEMM_ERR_HIP;
}

int gemm_attention_probs(const void* Q, const void* Kmat, int64_t batch, int64_t M, int64_t N,
                         int64_t D, int32_t dtype, int32_t k_layout, float scale, void* P,
                         int32_t p_dtype, void* stream) {
  const bool kn = k_layout == GEMM_B_KN;
  if (batch < 1 || M < 1 || N < 1 || N > 512 || D < 8 || D > 64 || D % 8 != 0 ||
      (kn && N % 8 != 0))
    return GEMM_ERR_SHAPE;
  if (!kn && k_layout != GEMM_B_NK) return GEMM_ERR_ARG;
  if (!std::isfinite(scale)) return GEMM_ERR_ARG;
  if (dtype != GEMM_BF16 && dtype != GEMM_F16) return GEMM_ERR_DTYPE;
  if (p_dtype != GEMM_F32 && p_dtype != GEMM_F16 && p_dtype != GEMM_BF16) return GEMM_ERR_DTYPE;
  if (!Q || !Kmat || !P) return GEMM_ERR_NULL;
  if (!aligned_to(Q, 16) || !aligned_to(Kmat, 16) || !aligned_to(P, elem_bytes(p_dtype)))
    return GEMM_ERR_ALIGN;
  // 32-bit byte offsets inside one item; the workgroup loop counts tiles in int64
  if (M * D * 2 >= (int64_t(1) << 31) || M * N * 4 >= (int64_t(1) << 31)) return GEMM_ERR_SHAPE;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return GEMM_ERR_NO_DEVICE;
  gemm_device_desc desc;
  if (device_desc(dev, &desc) != GEMM_OK) return GEMM_ERR_HIP;
  LaunchArgs a{};
  a.M = M;
  a.N = N;
  a.K = D;
  a.batch = batch;
  a.A = Q;
  a.sA = M * D;
  a.B = Kmat;
  a.sB = N * D;
  a.C = P;
  a.sC = M * N;
  a.epi.flags = 0;
  a.epi.scale = scale;
  a.epi.out_dtype = p_dtype == GEMM_F32 ? DT_F32 : p_dtype == GEMM_BF16 ? DT_BF16 : DT_F16;
  a.split = attention_workgroups(desc.cu_count);
  a.lda = D;
  a.ldb = kn ? N : D;
  a.ldc = N;
  const hipError_t err = launch_attention_probs(a, dtype == GEMM_BF16, kn,
                                                static_cast<hipStream_t>(stream));
  return err == hipSuccess ? GEMM_OK : GEMM_ERR_HIP;
}

int gemm_run_strided_batched_ws(const gemm_plan* p, int64_t batch, const void* A, int64_t sA,
                                const void* B, int64_t sB, const float* bias, const void* resid,
                                int64_t sR, void* C, int64_t sC, void* ws, int64_t ws_bytes,
                                void* stream) {
  if (!p) return GEMM_ERR_PLAN;
  if (batch < 1 || batch > 65535 || sA < 0 || sB < 0 || sC < 0 || sR < 0) return GEMM_ERR_ARG;
  if (!A || !B || !C) return GEMM_ERR_NULL;
  if (ws_bytes < 0 || (!ws && ws_bytes != 0)) return GEMM_ERR_ARG;
  const gemm_epilogue& e = p->epi;
  if ((e.flags & GEMM_EPI_BIAS) && !bias) return GEMM_ERR_NULL;
  if ((e.flags & GEMM_EPI_RESID) && !resid) return GEMM_ERR_NULL;
  const size_t ie = elem_bytes(p->dtype), oe = elem_bytes(e.out_dtype);
  if (!aligned_to(A, ie) || !aligned_to(B, ie) || !aligned_to(C, oe)) return GEMM_ERR_ALIGN;
  if ((e.flags & GEMM_EPI_BIAS) && !aligned_to(bias, 4)) return GEMM_ERR_ALIGN;
  if ((e.flags & GEMM_EPI_RESID) && !aligned_to(resid, oe)) return GEMM_ERR_ALIGN;
  if (ws && !aligned_to(ws, 256)) return GEMM_ERR_ALIGN;
  if (ws && ws_bytes < p->workspace_bytes) return GEMM_ERR_WORKSPACE;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return GEMM_ERR_HIP;
  if (dev != p->device) return GEMM_ERR_PLAN;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  if (poison_enabled()) {
    // debug aid (GEMM15_POISON): C starts as NaN, unless the residual shares its memory
    const char* c0 = static_cast<const char*>(C);
    const char* r0 = static_cast<const char*>(resid);
    const int64_t cspan = ((batch - 1) * sC + p->M * p->N) * static_cast<int64_t>(oe);
    const int64_t rspan = ((batch - 1) * sR + p->M * p->N) * static_cast<int64_t>(oe);
    const bool overlap = (e.flags & GEMM_EPI_RESID) && r0 < c0 + cspan && c0 < r0 + rspan;
    if (!overlap && aligned_to(C, 4) && (p->N * oe) % 4 == 0 && (sC * oe) % 4 == 0 &&
        poison_output(C, p->M, p->N, p->N, batch, sC, e.out_dtype, st) != hipSuccess)
      return GEMM_ERR_HIP;
  }
  // scratch for the plan's own configuration, or its workspace-free configuration
  const bool use_ws = p->workspace_bytes > 0 && ws != nullptr;
  const bool no_ws = p->workspace_bytes > 0 && !use_ws;
  if (no_ws && p->nows < 0) return GEMM_ERR_WORKSPACE;

  // The vector kernels need 16-byte aligned base pointers and batch strides.
  const bool a16 = aligned_to(A, 16) && aligned_to(B, 16) && aligned_to(C, 16) &&
                   (sA * ie) % 16 == 0 && (sB * ie) % 16 == 0 && (sC * oe) % 16 == 0 &&
                   (!(e.flags & GEMM_EPI_RESID) || (aligned_to(resid, 16) && (sR * oe) % 16 == 0));
  const auto& all = registry().all;
  const bool c16 = aligned_to(C, 16) && (p->N * oe) % 16 == 0 && (sC * oe) % 16 == 0 &&
                   (!(e.flags & GEMM_EPI_RESID) || (aligned_to(resid, 16) && (sR * oe) % 16 == 0));
  if (p->edge_m + p->edge_n > 0 && (use_ws || p->workspace_bytes == 0)) {
    // thin edges split off: operands not copied, C and the residual must start on
    // 16 bytes (their rows may have any length)
    const bool a_ok = (p->packed & 1) || (aligned_to(A, 16) && (sA * ie) % 16 == 0);
    const bool b_ok = (p->packed & 2) || (aligned_to(B, 16) && (sB * ie) % 16 == 0);
    const bool c_ok = aligned_to(C, 16) && (sC * oe) % 16 == 0 &&
                      (!(e.flags & GEMM_EPI_RESID) || (aligned_to(resid, 16) && (sR * oe) % 16 == 0));
    if (a_ok && b_ok && c_ok)
      return run_edges(p, batch, A, sA, B, sB, bias, resid, sR, C, sC, c16, ws, st);
  }
  if (p->packed && use_ws) {
    // operands that are not copied must still be 16-byte aligned for the kernel
    const bool a_ok = (p->packed & 1) || (aligned_to(A, 16) && (sA * ie) % 16 == 0);
    const bool b_ok = (p->packed & 2) || (aligned_to(B, 16) && (sB * ie) % 16 == 0);
    if (a_ok && b_ok) return run_packed(p, batch, A, sA, B, sB, bias, resid, sR, C, sC, c16, ws, st);
  }
  // The register-load streaming form reads A and B at any 2-byte alignment and any
  // batch stride; it stores C (and reads the residual) in 4- or 2-byte units.
  const KernelEntry& kp = all[p->config];
  const bool c4 = aligned_to(C, 4) && (sC * oe) % 4 == 0 &&
                  (!(e.flags & GEMM_EPI_RESID) || (aligned_to(resid, 4) && (sR * oe) % 4 == 0));
  int ci = p->fallback;
  if (!p->packed && kp.kind == KIND_K1 && !kp.vec_a && !kp.vec_b && c4) ci = p->config;
  else if (a16 && !p->packed) ci = no_ws ? p->nows : p->config;
  else if (a16 && no_ws) ci = p->nows;
  if (ci < 0) return GEMM_ERR_ALIGN;  // transposed B: 16-byte aligned operands required
  const KernelEntry& k = all[ci];
  if (p->split > 1 && ci == p->config && k.kind == KIND_MFMA16 && use_ws)
    return run_split_k(p, k, batch, A, sA, B, sB, bias, resid, sR, C, sC, ws, st);

  const int64_t tiles = ((p->M + k.bm - 1) / k.bm) * ((p->N + k.bn - 1) / k.bn);
  if (tiles > 0x7fffffff) return GEMM_ERR_SHAPE;
  if (k.kind == KIND_SIMPLE && (p->M + k.bm - 1) / k.bm > 65535) return GEMM_ERR_SHAPE;

  LaunchArgs la;
  la.M = p->M;
  la.N = p->N;
  la.K = p->K;
  la.batch = batch;
  la.A = A;
  la.sA = sA;
  la.B = B;
  la.sB = sB;
  la.C = C;
  la.sC = sC;
  la.sR = sR;
  la.epi.flags = e.flags;
  la.epi.scale = e.scale;
  la.epi.bias = bias;
  la.epi.resid = resid;
  la.epi.out_dtype = e.out_dtype;
  la.workspace = nullptr;
  la.workspace_bytes = 0;
  la.split = 1;
  if (ci == p->config && k.kind == KIND_K1) la.split = p->split;  // resident workgroups
  if (ci == p->config && k.kind == KIND_GEMV && use_ws) {
    la.split = p->split;
    la.workspace = ws;
    la.workspace_bytes = p->workspace_bytes;
  }
  la.lda = p->K;
  la.ldb = p->b_nk ? p->K : p->N;
  la.ldc = p->N;
  la.c_vec = (a16 && p->N % 8 == 0) ? 1 : 0;
  const hipError_t err = k.launch(la, st);
  return err == hipSuccess ? GEMM_OK : GEMM_ERR_HIP;
}

int gemm_run_strided_batched(const gemm_plan* p, int64_t batch, const void* A, int64_t sA,
                             const void* B, int64_t sB, const float* bias, const void* resid,
                             int64_t sR, void* C, int64_t sC, void* stream) {
  return gemm_run_strided_batched_ws(p, batch, A, sA, B, sB, bias, resid, sR, C, sC, nullptr, 0,
                                     stream);
}

int gemm_run_ws(const gemm_plan* p, const void* A, const void* B, const float* bias,
                const void* resid, void* C, void* ws, int64_t ws_bytes, void* stream) {
  if (!p) return GEMM_ERR_PLAN;
  return gemm_run_strided_batched_ws(p, 1, A, 0, B, 0, bias, resid, 0, C, 0, ws, ws_bytes, stream);
}

int gemm_run(const gemm_plan* p, const void* A, const void* B, const float* bias,
             const void* resid, void* C, void* stream) {
  if (!p) return GEMM_ERR_PLAN;
  return gemm_run_strided_batched_ws(p, 1, A, 0, B, 0, bias, resid, 0, C, 0, nullptr, 0, stream);
}

int gemm_run_noalloc(const gemm_plan* p, int64_t batch, const void* A, int64_t sA, const void* B,
                     int64_t sB, const float* bias, const void* resid, int64_t sR, void* C,
                     int64_t sC, void* stream) {
  if (!p) return GEMM_ERR_PLAN;
  if (p->workspace_bytes == 0)
    return gemm_run_strided_batched_ws(p, batch, A, sA, B, sB, bias, resid, sR, C, sC, nullptr, 0,
                                       stream);
  if (p->workspace_bytes > kScratchBytes) return GEMM_ERR_WORKSPACE;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return GEMM_ERR_HIP;
  if (dev != p->device) return GEMM_ERR_PLAN;
  void* ws = scratch_address(dev);
  if (!ws) return GEMM_ERR_HIP;
  return gemm_run_strided_batched_ws(p, batch, A, sA, B, sB, bias, resid, sR, C, sC, ws,
                                     kScratchBytes, stream);
}

int64_t gemm_noalloc_scratch_bytes(void) { return kScratchBytes; }

int64_t gemm_plan_workspace_bytes(const gemm_plan* p) {
  if (!p) return GEMM_ERR_PLAN;
  return p->workspace_bytes;
}

void gemm_plan_destroy(gemm_plan* p) { delete p; }

int gemm_last_error(void) { return t_last_error; }

const char* gemm_strerror(int s) {
  switch (s) {
    case GEMM_OK: return "success";
    case GEMM_ERR_SHAPE: return "invalid shape (a dimension < 1, or too large for the grid)";
    case GEMM_ERR_DTYPE: return "invalid element type or epilogue flags";
    case GEMM_ERR_NULL: return "a required pointer is NULL";
    case GEMM_ERR_ALIGN: return "a pointer is not aligned to its element size";
    case GEMM_ERR_NO_DEVICE: return "no HIP device is visible";
    case GEMM_ERR_HIP: return "a HIP runtime call or kernel launch failed";
    case GEMM_ERR_PLAN: return "NULL plan, or plan used on another device";
    case GEMM_ERR_NOMEM: return "out of memory while creating a plan";
    case GEMM_ERR_CONFIG: return "the requested configuration cannot run this problem";
    case GEMM_ERR_ARG: return "invalid argument";
    case GEMM_ERR_WORKSPACE:
      return "the workspace is smaller than the plan needs, or the plan cannot run without one";
  }
  return "unknown status";
}

int gemm_plan_describe(const gemm_plan* p, char* buf, size_t len) {
  if (!p) return GEMM_ERR_PLAN;
  return describe_plan(p, buf, len);
}

int gemm_select_layout(const gemm_device_desc* dev, int64_t M, int64_t N, int64_t K,
                       int32_t dtype, const gemm_epilogue* epi_in, int64_t batch_hint,
                       int32_t aligned16, int32_t b_layout, gemm_choice* out) {
  if (!dev || !out) return GEMM_ERR_NULL;
  if (b_layout != GEMM_B_KN && b_layout != GEMM_B_NK) return GEMM_ERR_ARG;
  const bool b_nk = b_layout == GEMM_B_NK;
  if (dev->cu_count < 1 || dev->lds_bytes < 1) return GEMM_ERR_ARG;
  const gemm_epilogue epi = norm_epi(epi_in);
  const int rc = check_problem(M, N, K, dtype, epi, batch_hint);
  if (rc) return rc;
  const Selection sel = choose(*dev, M, N, K, dtype, epi, batch_hint, aligned16 != 0, b_nk);
  const int cfg = sel.config;
  if (cfg < 0) return GEMM_ERR_CONFIG;
  const KernelEntry& k = registry().all[cfg];
  out->config = cfg;
  out->kind = k.kind;
  out->bm = k.bm;
  out->bn = k.bn;
  out->bk = k.bk;
  out->threads = k.threads;
  out->lds_bytes = k.lds_bytes;
  out->split = k.kind == KIND_GEMV ? gemv_split(k, N, K, batch_hint, *dev)
               : (k.kind == KIND_MFMA16 && !sel.packed && !b_nk)
                   ? tile_split(k, M, N, K, batch_hint, *dev)
                   : 1;
  out->workgroups = cfg_workgroups(k, M, N, k.kind == KIND_K1 ? k1_workgroups(k, *dev) : out->split,
                                   batch_hint);
  out->packed = sel.packed;
  return GEMM_OK;
}

int gemm_select(const gemm_device_desc* dev, int64_t M, int64_t N, int64_t K, int32_t dtype,
                const gemm_epilogue* epi, int64_t batch_hint, int32_t aligned16,
                gemm_choice* out) {
  return gemm_select_layout(dev, M, N, K, dtype, epi, batch_hint, aligned16, GEMM_B_KN, out);
}

int gemm_config_count(void) { return static_cast<int>(registry().all.size()); }

const char* gemm_config_name(int32_t i) {
  const auto& all = registry().all;
  if (i < 0 || i >= static_cast<int32_t>(all.size())) return nullptr;
  return all[i].name;
}

void gemm_cache_stats(int64_t* hits, int64_t* misses, int64_t* entries) {
  Cache& c = cache();
  std::lock_guard<std::mutex> lk(c.mu);
  if (hits) *hits = c.hits;
  if (misses) *misses = c.misses;
  if (entries) *entries = static_cast<int64_t>(c.map.size());
}

}  // extern "C"
