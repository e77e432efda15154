"""Build libv4attn.so (HIP for gfx950) in-tree, next to this file.

Usage: python -m long_context_attention_compress_amd.build  (or build() from Python).
Objects go to _build/ at the repository root; the shared library is written
into the package directory so that it travels with the source tree.
"""

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, 'csrc')
BUILD = os.path.join(ROOT, '_build')
LIB = os.path.join(PKG, 'libv4attn.so')

SOURCES = ['compress.hip', 'index.hip', 'attn.hip', 'noalloc.hip', 'abi.cpp']
ARCH = os.environ.get('V4A_OFFLOAD_ARCH', 'gfx950')
FLAGS = ['-O3', '-fPIC', '-std=c++17', f'--offload-arch={ARCH}', '-Wall', '-Wno-unused-function',
         '-Xclang', '-target-feature', '-Xclang', '-packed-fp32-ops',
         '-I', os.path.join(ROOT, 'include'), '-I', CSRC]


# Per-source extra flags. The indexer's MFMA results feed VALU arithmetic
# directly, so they are kept in ordinary VGPRs rather than accumulation
# registers (saving a register move per element).
EXTRA = {'index.hip': ['-mllvm', '-amdgpu-mfma-vgpr-form=1']}


def _hipcc():
    for c in (os.environ.get('HIPCC'), '/opt/rocm/bin/hipcc', shutil.which('hipcc')):
        if c and os.path.exists(c):
            return c
    raise RuntimeError('hipcc not found')


def _compile(src):
    obj = os.path.join(BUILD, os.path.basename(src) + '.o')
    lang = ['-x', 'hip'] if src.endswith('.hip') else []
    cmd = [_hipcc()] + FLAGS + EXTRA.get(src, []) + lang + ['-c', os.path.join(CSRC, src), '-o', obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = '\n'.join(l for l in (r.stdout + r.stderr).splitlines() if 'packed-fp32-ops' not in l)
    if r.returncode != 0:
        raise RuntimeError(f'compile failed: {src}\n{" ".join(cmd)}\n{out}')
    return obj, out


def build(verbose=True):
    os.makedirs(BUILD, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(len(SOURCES), 8)) as ex:
        results = list(ex.map(_compile, SOURCES))
    for obj, out in results:
        if out.strip() and verbose:
            print(out, file=sys.stderr)
    tmp = LIB + '.tmp'
    cmd = [_hipcc(), '-shared', f'--offload-arch={ARCH}', '-o', tmp] + [o for o, _ in results]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f'link failed\n{" ".join(cmd)}\n{r.stdout}{r.stderr}')
    os.replace(tmp, LIB)
    if verbose:
        print(f'built {LIB}', file=sys.stderr)
    return LIB


if __name__ == '__main__':
    build()
