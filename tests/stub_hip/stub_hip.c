/* A CPU stand-in for the HIP entry points liblighthouse.so imports, for host
 * tests without a GPU.  Kernel launches are not run: each is written to
 * stderr as one line (kernel, grid, block, dynamic LDS) and checked against
 * the MI355X limits (1024 threads per workgroup, 160 KiB of LDS per
 * workgroup, grid y and z below 65536, grid work-items in 32 bits).
 * Device pointers are never dereferenced by the host code, so callers may
 * pass any aligned address.  Built with a version script giving the symbols
 * the version the library was linked against. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

typedef int hipError_t;
typedef void *hipStream_t;
typedef void *hipEvent_t;
typedef struct { uint32_t x, y, z; } dim3;

#define MAX_FN 4096
static struct { const void *f; char name[200]; } fns[MAX_FN];
static int nfn;
static dim3 cfg_grid, cfg_block;
static size_t cfg_shm;
static hipStream_t cfg_stream;
static void *module_handle;

void **__hipRegisterFatBinary(const void *data) { (void)data; return &module_handle; }
void __hipRegisterFunction(void **m, const void *host_fn, char *dev_fn, const char *dev_name,
                           unsigned limit, void *tid, void *bid, dim3 *bd, dim3 *gd, int *ws) {
  (void)m; (void)dev_fn; (void)limit; (void)tid; (void)bid; (void)bd; (void)gd; (void)ws;
  if (nfn < MAX_FN) {
    fns[nfn].f = host_fn;
    strncpy(fns[nfn].name, dev_name, sizeof(fns[nfn].name) - 1);
    ++nfn;
  }
}
void __hipRegisterVar(void **m, void *var, char *hv, char *dv, int ext, size_t size, int c, int g) {
  (void)m; (void)var; (void)hv; (void)dv; (void)ext; (void)size; (void)c; (void)g;
}
void __hipUnregisterFatBinary(void **m) { (void)m; }

hipError_t __hipPushCallConfiguration(dim3 g, dim3 b, size_t shm, hipStream_t st) {
  cfg_grid = g; cfg_block = b; cfg_shm = shm; cfg_stream = st;
  return 0;
}
hipError_t __hipPopCallConfiguration(dim3 *g, dim3 *b, size_t *shm, hipStream_t *st) {
  *g = cfg_grid; *b = cfg_block; *shm = cfg_shm; *st = cfg_stream;
  return 0;
}

hipError_t hipLaunchKernel(const void *f, dim3 g, dim3 b, void **args, size_t shm,
                           hipStream_t st) {
  (void)args; (void)st;
  const char *name = "?";
  for (int i = 0; i < nfn; ++i)
    if (fns[i].f == f) name = fns[i].name;
  const uint64_t threads = (uint64_t)b.x * b.y * b.z;
  const int bad = threads == 0 || threads > 1024 || shm > 160 * 1024 || g.x == 0 || g.y == 0 ||
                  g.z == 0 || g.y > 65535 || g.z > 65535 ||
                  (uint64_t)g.x * b.x > 0xffffffffull;
  fprintf(stderr, "[launch] %s grid %u %u %u block %u %u %u shm %zu %s\n", name, g.x, g.y, g.z,
          b.x, b.y, b.z, shm, bad ? "BAD" : "ok");
  return 0;
}

hipError_t hipEventCreateWithFlags(hipEvent_t *e, unsigned flags) {
  (void)flags; *e = malloc(16); return 0;
}
hipError_t hipEventRecord(hipEvent_t e, hipStream_t s) { (void)e; (void)s; return 0; }
hipError_t hipFuncSetAttribute(const void *f, int attr, int v) { (void)f; (void)attr; (void)v; return 0; }
hipError_t hipGetDevice(int *d) { *d = 0; return 0; }
hipError_t hipGetLastError(void) { return 0; }
hipError_t hipGetSymbolAddress(void **p, const void *sym) { *p = (void *)sym; return 0; }
hipError_t hipStreamCreateWithFlags(hipStream_t *s, unsigned flags) {
  (void)flags; *s = malloc(16); return 0;
}
hipError_t hipStreamWaitEvent(hipStream_t s, hipEvent_t e, unsigned flags) {
  (void)s; (void)e; (void)flags; return 0;
}
