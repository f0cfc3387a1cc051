// The measured dispatch table (host only): which kernel a product takes at a
// given (type, N, K) and M, read once from a text file written by a sweep of
// every kernel on the device (llama.cpp PR 1632 "mulmat tune", Solutions
// items 3-4: a self-contained bench data file consulted at run time, with
// the choice between measured batch sizes interpolated, instead of a fixed
// "M >= 32" rule whose misplaced threshold costs tens of percent).
//
// File: MM_DISPATCH_TABLE if set, else dispatch_table.txt beside the
// library.  Lines "type N K M_lo M_hi variant" (type f32, f16, q4_0 or
// q4_0r; variant 1 narrow, 2 wide, 3 skinny MFMA), '#' starts a comment.
// The sweep measures M = 2^n and puts each crossover at the geometric mean
// of the two measured M on either side, so that an M between them takes the
// kernel of the nearer one in log M.  A missing file, a malformed line or a
// variant the type has no kernel for leaves that shape to the built-in
// rules.  MM_VERBOSE=1 prints the file read and every decision on stderr.
// MM_NARROW_MAX_M and MM_SPLIT_K, read with the table, override the narrow
// kernel's M range and the K split for experiments (plan.h).
#include "plan.h"

#include <dlfcn.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <mutex>
#include <string>
#include <vector>

#include "../../include/mm.h"

namespace qsg {

namespace {

struct Entry {
  int type;
  int64_t n, k, m_lo, m_hi;
  int variant;
};

std::once_flag g_once;
std::vector<Entry> g_table;
bool g_verbose = false;
int g_narrow_max_m = -1;   // MM_NARROW_MAX_M, -1 unset
int g_split_k = -1;        // MM_SPLIT_K, -1 unset

int type_of(const char* s) {
  if (!strcmp(s, "f32")) return MM_TYPE_F32;
  if (!strcmp(s, "f16")) return MM_TYPE_F16;
  if (!strcmp(s, "q4_0")) return MM_TYPE_Q4_0;
  if (!strcmp(s, "q4_0r")) return MM_TYPE_Q4_0R;
  return -1;
}

bool variant_ok(int type, int v) {
  if (v < 1 || v > 3) return false;
  if (type == MM_TYPE_F32 && v == 2) return false;     // no wide F32 kernel
  if (type == MM_TYPE_Q4_0R && v == 1) return false;   // no narrow kernel on repacked weights
  return true;
}

std::string default_path() {
  Dl_info info;
  if (dladdr(reinterpret_cast<void*>(&dispatch_table_variant), &info) && info.dli_fname) {
    std::string p(info.dli_fname);
    const size_t slash = p.rfind('/');
    return (slash == std::string::npos ? std::string(".") : p.substr(0, slash)) +
           "/dispatch_table.txt";
  }
  return "dispatch_table.txt";
}

// A positive integer from the environment, or -1 (unset or not a number).
int env_count(const char* name) {
  const char* v = getenv(name);
  if (!v || !v[0]) return -1;
  char* end = nullptr;
  const long x = strtol(v, &end, 10);
  if (*end || x < 0 || x > (1 << 20)) {
    if (g_verbose) fprintf(stderr, "[mm] %s=%s ignored\n", name, v);
    return -1;
  }
  return (int)x;
}

void load() {
  const char* v = getenv("MM_VERBOSE");
  g_verbose = v && v[0] && strcmp(v, "0") != 0;
  g_narrow_max_m = env_count("MM_NARROW_MAX_M");
  g_split_k = env_count("MM_SPLIT_K");
  if (g_split_k == 0) g_split_k = -1;
  if (g_verbose && (g_narrow_max_m >= 0 || g_split_k > 0))
    fprintf(stderr, "[mm] overrides: MM_NARROW_MAX_M %d, MM_SPLIT_K %d\n", g_narrow_max_m, g_split_k);
  const char* env = getenv("MM_DISPATCH_TABLE");
  const std::string path = env && env[0] ? std::string(env) : default_path();
  FILE* f = fopen(path.c_str(), "r");
  if (!f) {
    if (g_verbose) fprintf(stderr, "[mm] dispatch table %s: not found, built-in rules\n", path.c_str());
    return;
  }
  char line[512];
  int lineno = 0, bad = 0;
  while (fgets(line, sizeof line, f)) {
    ++lineno;
    char* hash = strchr(line, '#');
    if (hash) *hash = 0;
    char tname[16];
    long long n, k, lo, hi;
    int var;
    const int got = sscanf(line, "%15s %lld %lld %lld %lld %d", tname, &n, &k, &lo, &hi, &var);
    if (got <= 0) continue;                          // blank or comment
    const int t = got == 6 ? type_of(tname) : -1;
    if (t < 0 || n <= 0 || k <= 0 || lo < 1 || hi < lo || !variant_ok(t, var)) {
      ++bad;
      if (g_verbose) fprintf(stderr, "[mm] dispatch table %s:%d ignored\n", path.c_str(), lineno);
      continue;
    }
    g_table.push_back(Entry{t, n, k, lo, hi, var});
  }
  fclose(f);
  if (g_verbose)
    fprintf(stderr, "[mm] dispatch table %s: %zu entries, %d ignored\n", path.c_str(),
            g_table.size(), bad);
}

}  // namespace

int env_narrow_max_m() {
  std::call_once(g_once, load);
  return g_narrow_max_m;
}

int env_split_k() {
  std::call_once(g_once, load);
  return g_split_k;
}

int dispatch_table_variant(int type, int64_t M, int64_t N, int64_t K) {
  std::call_once(g_once, load);
  int v = 0;
  for (const Entry& e : g_table)
    if (e.type == type && e.n == N && e.k == K && M >= e.m_lo && M <= e.m_hi) {
      v = e.variant;
      break;
    }
  return v;
}

void dispatch_log(int type, int64_t M, int64_t N, int64_t K, int variant, bool from_table) {
  if (!g_verbose) return;
  fprintf(stderr, "[mm] type %d M %lld N %lld K %lld -> variant %d (%s)\n", type, (long long)M,
          (long long)N, (long long)K, variant, from_table ? "table" : "rules");
}

}  // namespace qsg
