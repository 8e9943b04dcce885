// Host-only parts of the library: the codebook and quantisation tables, and
// the planning of grids, splits and workspace sizes.  No device code lives
// here, so this file (with the C ABI) also builds on the CPU alone, with the
// kernel launchers stubbed, for the sanitizer check of the host logic.
#include <math.h>
#include <string.h>

#include "launch.h"

namespace qlora {

namespace {
int64_t cdiv(int64_t n, int64_t d) { return (n + d - 1) / d; }
}  // namespace

// ------------------------------------------------------------ tables

// Library copies of the codebooks (QLoRA Appendix E for NF4; the other
// types of the section 3 comparison as defined in codebooks.h).
const NF4Values& code_values(int code_type) {
  static NF4Values v[CODE_TYPES];
  static const bool filled = [] {
    for (int c = 0; c < CODE_TYPES; ++c) memcpy(v[c].v, kCodeValuesHost[c], sizeof(v[c].v));
    return true;
  }();
  (void)filled;
  return v[code_type];
}

// Decision thresholds between codes i and i+1 are the exact midpoints
// (NF4[i] + NF4[i+1]) / 2 (exact in double), rounded toward -inf to fp32 so
// that "x > thr" equals "x > midpoint" for every fp32 x; a tie (x equal to a
// midpoint) keeps the lower code.  Each bucket (width 1/16) holds at most one
// midpoint, since adjacent midpoints are more than 1/16 apart.  The bucket
// index is computed exactly from x; an x on the edge between two buckets
// gets the same code from either of them.
namespace {
// Set when a table builder finds a bucket holding two decision points (which
// the fixed codebooks never give); quantisation then refuses to run.
bool g_nf4_table_bad = false;
bool g_fine_table_bad = false;
}  // namespace

const QuantTable& quant_table() {
  static const QuantTable t = [] {
    QuantTable q;
    double mid[15];
    float thr[15];
    for (int i = 0; i < 15; ++i) {
      mid[i] = 0.5 * ((double)kCodeValuesHost[CODE_NF4][i] + (double)kCodeValuesHost[CODE_NF4][i + 1]);
      float f = (float)mid[i];
      if ((double)f > mid[i]) f = nextafterf(f, -INFINITY);
      thr[i] = f;
    }
    for (int b = 0; b < kBuckets; ++b) {
      const double lo = (b - 0.5) / 16.0 - 1.0, hi = (b + 0.5) / 16.0 - 1.0;
      uint32_t base = 0;
      float t_in = INFINITY;
      int inside = 0;
      for (int i = 0; i < 15; ++i) {
        if (mid[i] < lo) ++base;
        else if (mid[i] < hi) { t_in = thr[i]; ++inside; }
      }
      if (inside > 1) g_nf4_table_bad = true;  // cannot happen for the Appendix E values
      q.thr[b] = t_in;
      q.base[b] = base;
    }
    return q;
  }();
  return t;
}

// Spec of the finer quantisation table of a codebook (any type): its
// distinct values in increasing order (the smallest code for a repeated
// value, so +0 rather than -0), the exact midpoints between neighbours and
// those rounded toward -inf to fp32.  Checks once that no fine bucket holds
// two midpoints (true for all four codebooks: the closest midpoints, E3M0's
// around zero, are 2^-6 apart against a bucket width of 2^-9).
const CodeSpec& code_spec(int code_type) {
  static CodeSpec specs[CODE_TYPES];
  static const bool built = [] {
    for (int c = 0; c < CODE_TYPES; ++c) {
      const float* v = kCodeValuesHost[c];
      float vals[16];
      uint32_t codes[16];
      int n = 0;
      for (int i = 0; i < 16; ++i) {  // insertion into the sorted distinct list
        int j = 0;
        while (j < n && vals[j] < v[i]) ++j;
        if (j < n && vals[j] == v[i]) continue;  // repeated value (-0): keep the smaller code
        for (int k = n; k > j; --k) { vals[k] = vals[k - 1]; codes[k] = codes[k - 1]; }
        vals[j] = v[i];
        codes[j] = (uint32_t)i;
        ++n;
      }
      CodeSpec& sp = specs[c];
      memset(&sp, 0, sizeof(sp));
      sp.nmid = n - 1;
      for (int i = 0; i < n; ++i) sp.rank_code[i] = codes[i];
      for (int i = 0; i + 1 < n; ++i) {
        sp.mid[i] = 0.5 * ((double)vals[i] + (double)vals[i + 1]);
        float f = (float)sp.mid[i];
        if ((double)f > sp.mid[i]) f = nextafterf(f, -INFINITY);
        sp.thr[i] = f;
      }
      for (int b = 0; b < kFineBuckets; ++b) {
        const double lo = (b - 0.5) / kFineScale - 1.0, hi = (b + 0.5) / kFineScale - 1.0;
        int inside = 0;
        for (int i = 0; i < sp.nmid; ++i) inside += sp.mid[i] >= lo && sp.mid[i] < hi;
        if (inside > 1) g_fine_table_bad = true;
      }
    }
    return true;
  }();
  (void)built;
  return specs[code_type];
}

bool quant_tables_ok(int code_type) {
  if (code_type == CODE_INT8) return true;
  (void)quant_table();
  (void)code_spec(code_type);
  return code_type == CODE_NF4 ? !g_nf4_table_bad : !g_fine_table_bad;
}

// Int8 values k / 127: the fp64 quotient is correctly rounded and, since
// the binary expansion of k / 127 repeats every 7 bits, never lies on an fp32
// rounding boundary, so converting it to fp32 rounds k / 127 once.
const Int8Tables& int8_tables() {
  static const Int8Tables t = [] {
    Int8Tables q;
    for (int c = 0; c < 256; ++c) q.value[c] = (float)((double)(c >= 128 ? c - 256 : c) / 127.0);
    for (int k = -127; k < 127; ++k) {
      const double mid = 0.5 * ((double)q.value[k & 0xFF] + (double)q.value[(k + 1) & 0xFF]);
      float f = (float)mid;
      if ((double)f > mid) f = nextafterf(f, -INFINITY);
      q.thr[k + 127] = f;
    }
    return q;
  }();
  return t;
}

// ------------------------------------------------------- planning

int quantize_parts(int64_t numel) {
  const int64_t units = (numel + kQuantGridUnit - 1) / kQuantGridUnit;
  return (int)(units < 1 ? 1 : (units > kQuantMaxParts ? kQuantMaxParts : units));
}
int quantize_parts_batched(int64_t numel) {
  const int64_t unit = kQuantGridUnit * kQuantBatchUnits;
  const int64_t units = (numel + unit - 1) / unit;
  return (int)(units < 1 ? 1 : (units > kQuantMaxParts ? kQuantMaxParts : units));
}

// ------------------------------------------------ main-GEMM tile choice
// The 256 x 256 kernel runs one workgroup per CU.  Its tiles go in rounds of
// kCUs; when the last round would leave CUs idle, its R tiles are cut along
// the reduction into `split` ranges (split * R <= kCUs), whose fp32 partial
// tiles a fixup pass adds.  The older 128-wide kernels remain for shapes
// where even that leaves most of the chip idle.
SplitPlan plan_256(int64_t M, int64_t ncols, int64_t L) {
  SplitPlan p;
  p.tiles = (int)(cdiv(M, 256) * cdiv(ncols, 256));
  const int nkt = (int)(L >> 6);
  const int R = p.tiles % kCUs;
  int split = R > 0 ? kCUs / R : 1;
  if (split > nkt / 4) split = nkt / 4;  // at least four k-steps per range (the forward's ranges start on multiples of four)
  if (split < 2) {
    p.full = p.tiles;
    p.split = 1;
  } else {
    p.full = p.tiles - R;
    p.split = split;
  }
  return p;
}

// Rough time in units of one 256 x 256 tile on a CU.
MainTile pick_tile(int64_t M, int64_t ncols, int64_t L) {
  const SplitPlan p = plan_256(M, ncols, L);
  double best_t = (double)(p.full / kCUs) + (p.full % kCUs ? 1.0 : 0.0) +
                  (p.split > 1 ? 1.0 / p.split + 0.05 : 0.0);
  MainTile best = T256x256;
  struct Cand { MainTile t; int bm, bn; double cost; };
  const Cand cands[2] = {{T256x128, 256, 128, 0.56}, {T128x128, 128, 128, 0.30}};
  for (const Cand& c : cands) {
    const int64_t tiles = (int64_t)cdiv(M, c.bm) * cdiv(ncols, c.bn);
    const double waves = (double)((tiles + 2 * kCUs - 1) / (2 * kCUs));
    const double t = waves * c.cost * 2;
    if (t < best_t - 1e-9) { best_t = t; best = c.t; }
  }
  return best;
}

int skinny_splits(int64_t M, int64_t Q, int64_t L) {
  int64_t tiles = (int64_t)cdiv(M, 64) * cdiv(Q, 64);
  if (tiles < 1) tiles = 1;
  int64_t s = (512 + tiles - 1) / tiles;
  const int64_t max_s = L / SK_BK > 0 ? L / SK_BK : 1;
  if (s > max_s) s = max_s;
  if (s < 1) s = 1;
  return (int)s;
}
int tn_splits(int64_t M, int64_t P, int64_t Q) {
  int64_t tiles = (int64_t)cdiv(P, 128) * cdiv(Q, 64);
  if (tiles < 1) tiles = 1;
  int64_t s = (256 + tiles - 1) / tiles;  // about one workgroup per CU
  const int64_t max_s = M / TN_BK > 0 ? M / TN_BK : 1;
  if (s > max_s) s = max_s;
  if (s < 1) s = 1;
  if (s > 64) s = 64;
  return (int)s;
}
int gemv_splits(int64_t M, int64_t N, int64_t K) {
  const int64_t tiles = (int64_t)cdiv(N, G3_ROWS), nchunks = ((K >> 6) + G3_CB - 1) / G3_CB;
  // one workgroup per CU over the whole grid
  int64_t s = (kCUs + tiles - 1) / tiles;
  // keep the fp32 partials (S * M * N * 4 bytes, written and read once)
  // below about 1/4 of the packed weight (N * K / 2 bytes)
  const int64_t by_bytes = K / (32 * (M > 0 ? M : 1));
  if (s > by_bytes) s = by_bytes;
  if (s > nchunks) s = nchunks;  // every split holds at least one chunk
  return (int)(s < 1 ? 1 : s);
}
int xa_chunks(int64_t K) { return (int)((K + kXaChunk - 1) / kXaChunk); }
int64_t main_split_bytes(int64_t M, int64_t ncols, int64_t L) {
  if (pick_tile(M, ncols, L) != T256x256) return 0;
  return plan_256(M, ncols, L).part_floats() * 4;
}

int clip_parts(int64_t n) {
  const int64_t wgs = (n + kOptThreads * 4 - 1) / (kOptThreads * 4);
  return (int)(wgs < 1 ? 1 : (wgs > kOptMaxParts ? kOptMaxParts : wgs));
}

}  // namespace qlora
